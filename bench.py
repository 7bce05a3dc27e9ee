"""Benchmark: the synthetic dense decode step on one MI355X.

A step is one decode token's worth of weight-quantized GEMVs: 36 layers x
(q, k, v, o, gate, up, down) + lm_head, 4-bit asymmetric group-64 weights
(4.257 GB packed), bf16 activations, M = 1.  Inputs are resident in HBM
before timing starts.  Reported:
  value          whole-step algorithmic bytes / step time (GB/s)
  tok_per_s      equivalent decode tokens per second (1 / step time)
  m16            the same weights in one verification pass with a 16-row
                 activation tile per projection (skinny M = 16)
  roofline       the GEMV kernel: algorithmic bytes per launch / mean launch
                 duration (HIP events on the launch stream) vs 8 TB/s
  cpu_baseline   the CPU oracle on a bounded sample of the same step

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("qgemv achieved HBM GB/s (% of MI355X peak) + equiv. decode tok/s, M=1 and M=16")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources that decide what the decode-step kernel reads and writes: the
# kernel, the shared helpers, and the C ABI that builds its work list
STEP_SOURCES = ("capi.hip", "q4_gemv.hip", "qg_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_weight_decode_dequant_amd", "csrc")
    for name in STEP_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % kernel)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


STEP_KERNEL = "q4_gemv_kernel<true, 1, 8>"
COPY_BYTES = 1 << 30
PLAIN_READ_BYTES = 4 << 30   # larger than every cache level


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def summarize_pmc(fetch_csv: str, write_csv: str, out_json: str, command: str):
    """Turn two rocprofv3 --pmc CSVs (FETCH_SIZE, then WRITE_SIZE) of a
    --traffic-pass run into HBM bytes per launch of the decode-step kernel,
    each counter scaled by what it reads for the plain 1 GiB copy."""
    def per_kernel(path, counter):
        vals = {}
        for r in _csv_rows(path):
            if _col(r, "Counter_Name", "counter_name") != counter:
                continue
            name = _col(r, "Kernel_Name", "kernel_name")
            vals.setdefault(name, []).append(float(_col(r, "Counter_Value", "counter_value")))
        return vals

    def pick(vals, pred):
        keys = [k for k in vals if pred(k)]
        if not keys:
            raise SystemExit("kernel not found in counters: %s" % sorted(vals))
        v = vals[keys[0]]
        return sum(v) / len(v), keys[0]

    def pick_copy(vals):
        # the calibration copy is the largest copy dispatch of the pass (the
        # input uploads also run small copy kernels)
        best = None
        for k, v in vals.items():
            if "copy" in k.lower() or "elementwise" in k.lower():
                m = max(v)
                if best is None or m > best[0]:
                    best = (m, k)
        if best is None:
            raise SystemExit("copy kernel not found in counters")
        return best

    out = {"command": command, "kernel_source_hash": kernel_source_hash()}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        step_kib, step_name = pick(vals, lambda k: STEP_KERNEL in k)
        copy_kib, copy_name = pick_copy(vals)
        factor = copy_kib * 1024 / COPY_BYTES
        out[counter] = {"step_kernel": step_name, "step_kib_per_dispatch": step_kib,
                        "copy_kernel": copy_name, "copy_kib_per_dispatch": copy_kib,
                        "copy_factor": factor, "step_bytes_scaled": step_kib * 1024 / factor}
    out["hbm_bytes_per_launch"] = int(out["FETCH_SIZE"]["step_bytes_scaled"] +
                                      out["WRITE_SIZE"]["step_bytes_scaled"])
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def _pmc_dispatches(path, counter):
    """{kernel name: [counter value per dispatch, in dispatch order]}."""
    rows = []
    for r in _csv_rows(path):
        if _col(r, "Counter_Name", "counter_name") != counter:
            continue
        rows.append((int(_col(r, "Dispatch_Id", "dispatch_id")), _col(r, "Kernel_Name", "kernel_name"),
                     float(_col(r, "Counter_Value", "counter_value"))))
    out = {}
    for _, name, v in sorted(rows):
        out.setdefault(name, []).append(v)
    return out


def _manifest_match(disp, manifest):
    """Pair the manifest entries of each kernel, in order, with that kernel's
    last dispatches (the counter pass launches each measured kernel after any
    incidental use of it, such as copies during set-up); returns
    [(entry, kernel name, value)] in manifest order."""
    names = {}
    for ent in manifest:
        hit = [k for k in disp if ent["kernel"] in k]
        if len(hit) != 1:
            raise SystemExit("kernel %r matches %d dispatch names" % (ent["kernel"], len(hit)))
        names.setdefault(hit[0], []).append(ent)
    pos = {}
    for name, ents in names.items():
        if len(disp[name]) < len(ents):
            raise SystemExit("too few dispatches of %r" % name)
        pos[name] = len(disp[name]) - len(ents)
    out = []
    for ent in manifest:
        name = [k for k in disp if ent["kernel"] in k][0]
        out.append((ent, name, disp[name][pos[name]]))
        pos[name] += 1
    return out


def summarize_counters(fetch_csv: str, write_csv: str, manifest_json: str, out_md: str,
                       command: str):
    """HBM traffic of every hot kernel from two rocprofv3 --pmc runs of
    `bench.py --counter-pass` (FETCH_SIZE, then WRITE_SIZE), each counter
    scaled by what it reads for two reference kernels of known size: a plain
    1 GiB read (the library's qg_plain_read) and torch's 1 GiB device copy.
    Writes a markdown table against the algorithmic bytes of each launch, and
    the decode-step kernel's figure to profiles/traffic_q4_gemv_step.json."""
    with open(manifest_json) as f:
        man = json.load(f)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _pmc_dispatches(path, counter)
        res[counter] = _manifest_match(disp, man["kernels"])
    cal = {}
    for counter, kind in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
        for ent, name, kib in res[counter]:
            if ent.get("calibration"):
                cal.setdefault(counter, {})[ent["calibration"]] = (
                    kib * 1024 / ent[kind] if ent[kind] else None, name, kib)
    f_read = cal["FETCH_SIZE"]["plain_read"][0]
    f_copy_r = cal["FETCH_SIZE"]["copy"][0]
    f_write = cal["WRITE_SIZE"]["copy"][0]
    lines = ["# HBM traffic per launch of the hot-path kernels (rocprofv3 counters)", "",
             "MI355X (gfx950), one GPU. Kernel sources hash `%s` (sha256 over every file "
             "under csrc/, as bench.py computes it)." % all_sources_hash(), "",
             "Commands (one counter per run):", "",
             "```", command, "```", "",
             "Calibration: FETCH_SIZE reads %.4f x the bytes of a plain 1 GiB read "
             "(`qg_plain_read`, non-temporal 16-byte loads) and %.4f x the bytes read by "
             "torch's 1 GiB device copy; WRITE_SIZE reads %.4f x the bytes that copy writes. "
             "Each kernel's counters below are divided by these factors (read: the plain-read "
             "factor; write: the copy factor)." % (f_read, f_copy_r, f_write), "",
             "| kernel | launch | algorithmic read (B) | counted read (B) | ratio | "
             "algorithmic write (B) | counted write (B) | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    rows = []
    for (ent, name, fk), (_, _, wk) in zip(res["FETCH_SIZE"], res["WRITE_SIZE"]):
        if ent.get("calibration"):
            continue
        rd = fk * 1024 / f_read
        wr = wk * 1024 / f_write
        rows.append({"kernel": ent["kernel"], "what": ent["what"], "algorithmic_read": ent["read"],
                     "counted_read": rd, "algorithmic_write": ent["write"], "counted_write": wr})
        lines.append("| `%s` | %s | %d | %d | %.4f | %d | %d | %.3f |" % (
            ent["kernel"], ent["what"], ent["read"], rd, rd / ent["read"], ent["write"], wr,
            wr / ent["write"] if ent["write"] else float("nan")))
    lines += ["", "Raw counter values (KiB per dispatch) are in the CSVs of the same commands; "
              "counted bytes = raw KiB x 1024 / factor."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    step = [r for r in rows if r["kernel"] == STEP_KERNEL]
    if step:
        s = step[0]
        rec = {"command": command, "kernel_source_hash": kernel_source_hash(),
               "FETCH_SIZE": {"step_kernel": STEP_KERNEL, "plain_read_factor": f_read,
                              "copy_read_factor": f_copy_r,
                              "step_bytes_scaled": s["counted_read"]},
               "WRITE_SIZE": {"step_kernel": STEP_KERNEL, "copy_factor": f_write,
                              "step_bytes_scaled": s["counted_write"]},
               "hbm_bytes_per_launch": int(s["counted_read"] + s["counted_write"])}
        with open(os.path.join(ROOT, "profiles", "traffic_q4_gemv_step.json"), "w") as f:
            json.dump(rec, f, indent=1)


MI355X_CUS, MI355X_SIMDS, MI355X_XCDS = 256, 1024, 8


def summarize_sq(csvs, manifest_json: str, out_md: str, command: str):
    """Per-launch SQ / TCC counters of `bench.py --counter-pass` runs (one
    rocprofv3 --pmc run per CSV, each with GRBM_GUI_ACTIVE), with the
    derived figures (GPU cycles = GRBM_GUI_ACTIVE per XCD): VALU busy =
    SQ_ACTIVE_INST_VALU / CUs / GPU cycles, MFMA
    busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / GPU cycles, LDS active =
    SQ_ACTIVE_INST_LDS / CUs / GPU cycles, and instruction counts per 1 KB of
    algorithmic read bytes."""
    with open(manifest_json) as f:
        man = [e for e in json.load(f)["kernels"] if not e.get("calibration")]
    vals = [dict() for _ in man]
    counters = []
    for path in csvs:
        rows = _csv_rows(path)
        for c in sorted({_col(r, "Counter_Name", "counter_name") for r in rows}):
            disp = _pmc_dispatches(path, c)
            try:
                hits = _manifest_match(disp, man)
            except SystemExit:
                continue
            if c not in counters:
                counters.append(c)
            for i, (_, _, v) in enumerate(hits):
                vals[i]["%s@%s" % (c, path)] = v
    lines = ["# SQ / TCC counters per launch of the hot-path kernels", "",
             "MI355X (gfx950), one GPU. Kernel sources hash `%s`." % all_sources_hash(), "",
             "Commands (one counter set per run, each with GRBM_GUI_ACTIVE for the busy "
             "percentages of that run):", "", "```", command, "```", ""]
    derived = []
    for i, ent in enumerate(man):
        row = {"kernel": ent["kernel"], "what": ent["what"]}
        kb = ent["read"] / 1024.0
        for path in csvs:
            g = vals[i].get("GRBM_GUI_ACTIVE@%s" % path)
            if g:
                # rocprofv3 sums the counter over its 8 instances (one per
                # XCD); the busy percentages use the per-XCD cycle count
                g = g / MI355X_XCDS
            for c in counters:
                v = vals[i].get("%s@%s" % (c, path))
                if v is None or c == "GRBM_GUI_ACTIVE":
                    continue
                row[c] = v
                if g:
                    if c == "SQ_ACTIVE_INST_VALU":
                        row["VALU busy %"] = 100 * v / MI355X_CUS / g
                    elif c == "SQ_VALU_MFMA_BUSY_CYCLES":
                        row["MFMA busy %"] = 100 * v / MI355X_SIMDS / g
                    elif c == "SQ_ACTIVE_INST_LDS":
                        row["LDS active %"] = 100 * v / MI355X_CUS / g
                    elif c == "SQ_LDS_BANK_CONFLICT":
                        row["LDS bank conflict %"] = 100 * v / MI355X_CUS / g
                if c.startswith("SQ_INSTS_"):
                    row[c + " per KB"] = v / kb
            if g:
                row["GPU cycles"] = g
        derived.append(row)
    keys = []
    for r in derived:
        for k in r:
            if k not in ("kernel", "what") and k not in keys:
                keys.append(k)
    lines.append("| kernel | launch | " + " | ".join(keys) + " |")
    lines.append("|---|---|" + "---|" * len(keys))
    for r in derived:
        cells = []
        for k in keys:
            v = r.get(k)
            cells.append("" if v is None else ("%.1f" % v if abs(v) < 1e4 else "%.4g" % v))
        lines.append("| `%s` | %s | %s |" % (r["kernel"], r["what"], " | ".join(cells)))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def all_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_weight_decode_dequant_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_pass(manifest_path: str, seed: int = 0):
    """Launch every measured hot-path kernel once, plus the two calibration
    kernels, and write the manifest: per launch, in launch order, the kernel
    and its algorithmic read and write bytes (for --summarize-counters)."""
    import torch
    import quantized_weight_decode_dequant_amd as pkg
    from quantized_weight_decode_dequant_amd import _lib, roofline, synth, weights, workloads
    assert torch.cuda.is_available(), "the counter pass needs a GPU"
    pkg.raw()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    man = []

    def add(kernel, what, read, write, calibration=None):
        e = {"kernel": kernel, "what": what, "read": int(read), "write": int(write)}
        if calibration:
            e["calibration"] = calibration
        man.append(e)

    Q4 = pkg.FMT_Q4_ASYM_G64
    step = workloads.build_decode_step(seed, log=log)
    wbytes = sum(roofline.Q4_BYTES_PER_WEIGHT * g.N * g.K for g in step.gemvs)
    sumK = sum(g.K for g in step.gemvs)
    sumN = sum(g.N for g in step.gemvs)
    plan = pkg.qg_batch_plan_build(Q4, 1, [(g.packed, g.N, g.K, g.x, g.y) for g in step.gemvs])
    torch.cuda.synchronize()
    pkg.qg_batch_run(plan)
    add(STEP_KERNEL, "decode step, 253 Q4 GEMVs, M=1, one launch", wbytes + 2 * sumK, 2 * sumN)
    for M, kern in ((16, "q4_skinny_stream_kernel<true, 1>"), (32, "q4_skinny_stream_kernel<true, 2>")):
        Xs = [workloads.verification_tile(seed, g, M) for g in step.gemvs]
        Ys = [torch.empty((M, g.N), dtype=torch.bfloat16, device=dev) for g in step.gemvs]
        planM = pkg.qg_batch_plan_build(Q4, M, [(g.packed, g.N, g.K, X, Y)
                                                for g, X, Y in zip(step.gemvs, Xs, Ys)])
        torch.cuda.synchronize()
        pkg.qg_batch_run(planM)
        add(kern, "verification pass, 253 Q4 products, M=%d, one launch" % M,
            wbytes + 2 * M * sumK, 2 * M * sumN)
        torch.cuda.synchronize()
        del Xs, Ys, planM
    del plan, step
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    for N, K in ((12288, 4096), (4096, 12288)):
        wl = workloads.Int8Verify(seed, N, K, copies=1)
        torch.cuda.synchronize()
        wl.quantize()
        add("had32_quant_kernel", "Hadamard-32 + int8 quant, 16 x %d" % K,
            2 * 16 * K + K, 16 * K + 4 * 16)
        wl.gemm()
        add("q8_skinny_kernel<1, %d, false>" % (2 if K == 4096 else 3),
            "int8 x int8 group-32, M=16, %d -> %d" % (K, N),
            roofline.Q8_BYTES_PER_WEIGHT * N * K + 16 * K + 4 * 16, 2 * 16 * N)
        torch.cuda.synchronize()
        del wl

    H, F, E, k = 7168, 2048, 384, 16
    eb = roofline.MXFP4_BYTES_PER_WEIGHT * H * F
    moe = workloads.MoeLayer(seed, E, H, F, k, routes=1)
    torch.cuda.synchronize()
    moe.run()
    add("qg::moe_gate_up_kernel", "MXFP4 MoE, one token: gate/up + SwiGLU of 16 experts",
        2 * k * eb + 2 * H, 4 * k * F)
    add("qg::moe_down_fused_kernel", "MXFP4 MoE, one token: down + combine of 16 experts",
        k * eb + 4 * k * F, 2 * H)
    torch.cuda.synchronize()
    del moe
    T = 16
    moet = workloads.MoeLayer(seed, E, H, F, k, routes=1, T=T)
    torch.cuda.synchronize()
    moet.run()
    dist = moet.distinct_experts()
    P = T * k
    add("moe_t_gate_up_kernel", "MXFP4 MoE, 16 positions: gate/up of %d distinct experts" % dist,
        2 * dist * eb + 2 * T * H, 4 * P * F)
    add("moe_t_down_kernel", "MXFP4 MoE, 16 positions: down of %d distinct experts" % dist,
        dist * eb + 4 * P * F, 4 * P * H)
    add("moe_combine_kernel", "MXFP4 MoE, 16 positions: combine", 4 * P * H, 2 * T * H)
    torch.cuda.synchronize()
    del moet
    torch.cuda.empty_cache()

    NH, KH = 151936, 4096
    gq = torch.Generator(device="cuda")
    gq.manual_seed(seed)
    qcodes = torch.randint(-128, 128, (NH, KH), dtype=torch.int8, device="cuda", generator=gq)
    qscales = (torch.rand(NH, dtype=torch.float32, device="cuda", generator=gq) + 0.5) * 2.0 ** -10
    qpacked = _lib.qgemv_pack(_lib.FMT_Q8_ROW, NH, KH, qcodes, qscales)
    del qcodes, qscales
    qx = weights.to_device(synth.activations(seed, 1, KH)[0], "cuda")
    qy = torch.empty(NH, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    _lib.qgemv_run(_lib.FMT_Q8_ROW, qpacked, NH, KH, qx, y=qy)
    add("q8row_gemv_kernel", "weight-only int8 head 4096 -> 151936", NH * KH + 4 * NH + 2 * KH,
        2 * NH)
    torch.cuda.synchronize()
    del qpacked

    # single skinny calls that span several staged K segments
    for name, N, K, M, kern in (("gate", 12288, 4096, 32, "q4_skinny_kernel<2, 1>"),
                                ("down", 4096, 12288, 16, "q4_skinny_kernel<1, 2>"),
                                ("down", 4096, 12288, 32, "q4_skinny_kernel<2, 1>")):
        m4 = synth.q4_matrix(seed, N, K, item=7)
        p4 = weights.pack_q4(m4, "cuda")
        del m4
        X4 = weights.to_device(synth.activations(seed + 1, M, K, item=7), "cuda")
        Y4 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        _lib.qgemm_skinny_run(Q4, p4, M, N, K, X4, Y=Y4)
        add(kern, "single Q4 skinny product %s %d -> %d, M=%d" % (name, K, N, M),
            roofline.Q4_BYTES_PER_WEIGHT * N * K + 2 * M * K, 2 * M * N)
        torch.cuda.synchronize()
        del p4, X4, Y4

    # one layer's seven affine verification products (3-bit g64, M = 16), one launch
    M3, B3, G3 = 16, 3, 64
    f3 = _lib.affine_format(B3, G3)
    g3 = torch.Generator(device="cuda")
    g3.manual_seed(seed + 30)
    ents, rd3, wr3 = [], 0, 0
    for name, k_in, n_out in synth.DECODE_PROJECTIONS:
        c3 = torch.randint(0, 1 << B3, (n_out, k_in), dtype=torch.uint8, device="cuda", generator=g3)
        s3 = ((torch.rand(n_out, k_in // G3, device="cuda", generator=g3) + 0.05) * 0.02 * 15 /
              ((1 << B3) - 1)).half().view(torch.int16)
        b3 = (torch.randn(n_out, k_in // G3, device="cuda", generator=g3) * 0.01).half().view(torch.int16)
        p3 = _lib.qgemv_pack(f3, n_out, k_in, c3, s3, b3)
        del c3, s3, b3
        X3 = weights.to_device(synth.activations(seed + 1, M3, k_in, item=len(ents)), "cuda")
        Y3 = torch.empty((M3, n_out), dtype=torch.bfloat16, device="cuda")
        ents.append((p3, n_out, k_in, X3, Y3))
        rd3 += n_out * k_in * (B3 / 8 + 4 / G3) + 2 * M3 * k_in
        wr3 += 2 * M3 * n_out
    plan3 = pkg.qg_batch_plan_build(f3, M3, ents)
    torch.cuda.synchronize()
    pkg.qg_batch_run(plan3)
    add("affine_skinny_kernel<true, 3, 2, 1, false>",
        "affine 3-bit g64 verification, one layer's 7 products, M=16, one launch", rd3, wr3)
    torch.cuda.synchronize()
    del ents, plan3

    NA, KA, GA = 262144, 8192, 64
    for bits in (2, 3):
        fa = _lib.affine_format(bits, GA)
        ga = torch.Generator(device="cuda")
        ga.manual_seed(seed + bits)
        acodes = torch.randint(0, 1 << bits, (NA, KA), dtype=torch.uint8, device="cuda", generator=ga)
        asc = ((torch.rand(NA, KA // GA, device="cuda", generator=ga) + 0.05) * 0.02 * 15 /
               ((1 << bits) - 1)).half().view(torch.int16)
        abi = (torch.randn(NA, KA // GA, device="cuda", generator=ga) * 0.01).half().view(torch.int16)
        apacked = _lib.qgemv_pack(fa, NA, KA, acodes, asc, abi)
        del acodes, asc, abi
        ax = weights.to_device(synth.activations(seed, 1, KA)[0], "cuda")
        ay = torch.empty(NA, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        _lib.qgemv_run(fa, apacked, NA, KA, ax, y=ay)
        add("affine_gemv_kernel<false, %d, 2," % bits, "affine %d-bit g64 GEMV 8192 -> 262144" % bits,
            NA * KA * (bits / 8 + 4 / GA) + 2 * KA, 2 * NA)
        torch.cuda.synchronize()
        del apacked

    # calibration: a plain read and a device copy of 1 GiB each
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    pkg.qg_plain_read(src, sink, 1024)
    add("plain_read_kernel", "calibration: plain read of 1 GiB", COPY_BYTES, 0,
        calibration="plain_read")
    dst.copy_(src)
    add("copyBuffer", "calibration: torch device copy of 1 GiB", COPY_BYTES, COPY_BYTES,
        calibration="copy")
    torch.cuda.synchronize()
    with open(manifest_path, "w") as f:
        json.dump({"kernels": man}, f, indent=1)
    log("counter pass: %d launches recorded in %s" % (len(man), manifest_path))


def summarize_trace(stats_csv: str, command: str, trace_csv: str = None, timed=None):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv;
    with the dispatch trace and the (first, count) of the timed launches that
    bench.py reports, also the mean duration of exactly those launches of the
    decode-step kernel."""
    rows = _csv_rows(stats_csv)
    print("Command: `%s`\n" % command)
    if trace_csv and timed:
        first, count = timed
        step = sorted((int(_col(r, "Dispatch_Id")), int(_col(r, "Start_Timestamp")),
                       int(_col(r, "End_Timestamp")))
                      for r in _csv_rows(trace_csv) if STEP_KERNEL in _col(r, "Kernel_Name"))
        win = step[first:first + count]
        mean_us = sum(e - b for _, b, e in win) / len(win) / 1e3
        print("Decode-step kernel `%s`: %d dispatches in the trace; the %d timed ones "
              "(dispatches %d..%d of the kernel) average %.2f us.\n" % (
                  STEP_KERNEL, len(step), len(win), first, first + len(win) - 1, mean_us))
    print("| kernel | calls | average (us) | min (us) | max (us) | share |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = _col(r, "Name", "KernelName", "Kernel_Name")
        print("| `%s` | %s | %.2f | %.2f | %.2f | %.2f%% |" % (
            name[:90], _col(r, "Calls"), float(_col(r, "AverageNs")) / 1e3,
            float(_col(r, "MinNs")) / 1e3, float(_col(r, "MaxNs")) / 1e3,
            float(_col(r, "Percentage"))))


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return "%s, %d logical CPUs" % (line.split(":", 1)[1].strip(), os.cpu_count() or 0)
    except OSError:
        pass
    return "unknown, %d logical CPUs" % (os.cpu_count() or 0)


def cpu_baseline(step, budget_s: float):
    """The oracle, as it stands, on the first GEMVs of the step until the time
    budget is spent (one thread; input generation is not timed)."""
    import oracle
    from quantized_weight_decode_dequant_amd import roofline, synth
    done_bytes, names, elapsed = 0.0, [], 0.0
    for item, name, N, K in synth.decode_step_shapes():
        m = synth.q4_matrix(step.seed, N, K, item=item)
        x = synth.activations(step.seed, 1, K, item=item)
        t = time.perf_counter()
        oracle.q4_gemm(m.codes, m.scales, m.biases, x)
        elapsed += time.perf_counter() - t
        done_bytes += roofline.q4_gemm_bytes(1, N, K)
        names.append(name)
        if elapsed >= budget_s:
            break
    gbs = done_bytes / elapsed / 1e9
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "tok_per_s": round(gbs * 1e9 / step.algorithmic_bytes(1), 6),
        "cores": 1,
        "kind": "oracle",
        "sample": "first %d GEMVs of the decode step (%s .. %s), %.3f GB algorithmic, %.1f s" % (
            len(names), names[0], names[-1], done_bytes / 1e9, elapsed),
    }


def cpu_baseline_all_cores(step, budget_s: float, threads: int):
    """The oracle, as it stands, on every host core the box gives this job:
    each GEMV's output rows are split into `threads` slices computed by
    concurrent oracle calls (the oracle releases the interpreter while it
    runs).  Same GEMVs as the one-thread figure, until the budget is spent."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from quantized_weight_decode_dequant_amd import roofline, synth
    done_bytes, n, elapsed = 0.0, 0, 0.0
    with ThreadPoolExecutor(threads) as pool:
        for item, name, N, K in synth.decode_step_shapes():
            m = synth.q4_matrix(step.seed, N, K, item=item)
            x = synth.activations(step.seed, 1, K, item=item)
            cuts = [N * i // threads for i in range(threads + 1)]
            t = time.perf_counter()
            list(pool.map(lambda j: oracle.q4_gemm(m.codes[cuts[j]:cuts[j + 1]],
                                                   m.scales[cuts[j]:cuts[j + 1]],
                                                   m.biases[cuts[j]:cuts[j + 1]], x),
                          range(threads)))
            elapsed += time.perf_counter() - t
            done_bytes += roofline.q4_gemm_bytes(1, N, K)
            n += 1
            if elapsed >= budget_s:
                break
    gbs = done_bytes / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s",
            "tok_per_s": round(gbs * 1e9 / step.algorithmic_bytes(1), 6),
            "cores": threads, "kind": "oracle",
            "sample": "first %d GEMVs of the decode step, output rows split over %d threads, "
                      "%.3f GB algorithmic, %.1f s" % (n, threads, done_bytes / 1e9, elapsed)}


def _split_rows(fn, N: int, threads: int, pool):
    """fn(r0, r1) for `threads` contiguous row slices, concurrently (the
    oracle releases the interpreter while it runs)."""
    cuts = [N * i // threads for i in range(threads + 1)]
    return list(pool.map(lambda j: fn(cuts[j], cuts[j + 1]), range(threads)))


def _timed(fn):
    t = time.perf_counter()
    fn()
    return time.perf_counter() - t


def cpu_baseline_configs(seed: int, threads: int):
    """The oracle, as it stands, on the other workloads of the path, timed
    whole on one thread and on `threads` threads (output rows, or experts,
    split over concurrent oracle calls); input generation is not timed.
      cfg1  the single 4-bit g64 GEMV 4096 x 4096, M = 1
      cfg4  the int8 verification at M = 16: Hadamard-32 + int8 quantization
            and the int8 x int8 group-32 product, for 4096 -> 12288 and
            12288 -> 4096
      cfg5  the MXFP4 MoE layer for one token: 16 of 384 experts (7168 x 2048)
      cfg3  the verification pass over the decode step's 253 projections at
            M = 16 and 32, extrapolated (in proportion to the weights, which
            fix the oracle's multiply-adds at a given M) from one timed
            decoder layer (q, k, v, o, gate, up, down) on `threads` threads;
            the config-1 matrix at M = 16 and 32 is timed beside it."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from quantized_weight_decode_dequant_amd import roofline, synth
    out = {}
    with ThreadPoolExecutor(threads) as pool:
        # cfg1
        m = synth.q4_matrix(seed, 4096, 4096)
        x = synth.activations(seed, 1, 4096)
        one = _timed(lambda: oracle.q4_gemm(m.codes, m.scales, m.biases, x))
        allc = _timed(lambda: _split_rows(lambda a, b: oracle.q4_gemm(
            m.codes[a:b], m.scales[a:b], m.biases[a:b], x), 4096, threads, pool))
        b = roofline.q4_gemm_bytes(1, 4096, 4096)
        out["cfg1_q4_gemv_4096x4096_m1"] = {
            "one_thread_s": round(one, 4), "all_cores_s": round(allc, 4),
            "one_thread_GBs": round(b / one / 1e9, 4), "all_cores_GBs": round(b / allc / 1e9, 4),
            "algorithmic_bytes": int(b)}
        # cfg4
        rows = {}
        for N, K in ((12288, 4096), (4096, 12288)):
            w = synth.q8_matrix(seed, N, K)
            X = synth.q8_activations(seed, 16, K)
            signs = synth.rotation_signs(seed, K)
            res = {}
            tq = _timed(lambda: res.setdefault("q", oracle.had32_quant(X, signs)))
            q, sx = res["q"]
            tg = _timed(lambda: oracle.q8_gemm(w.qw, w.sw, q, sx))
            tga = _timed(lambda: _split_rows(lambda a, c: oracle.q8_gemm(
                w.qw[a:c], w.sw[a:c], q, sx), N, threads, pool))
            bt = roofline.hadamard_quant_bytes(16, K) + roofline.q8_gemm_bytes(16, N, K)
            rows["%dx%d" % (K, N)] = {
                "hadamard_quant_s": round(tq, 4), "gemm_one_thread_s": round(tg, 4),
                "gemm_all_cores_s": round(tga, 4),
                "one_thread_GBs": round(bt / (tq + tg) / 1e9, 4),
                "all_cores_GBs": round(bt / (tq + tga) / 1e9, 4), "algorithmic_bytes": int(bt)}
        out["cfg4_int8_verification_m16"] = rows
        # cfg5: only the 16 selected experts are generated (the oracle reads
        # nothing else); ids renumbered into that pool
        H, F, k = 7168, 2048, 16
        ids, wts = synth.router(seed, 384, k)
        ex = [synth.expert(seed, int(e), H, F) for e in ids]
        st = lambda f, sel: np.stack([f(ex[i]) for i in sel])  # noqa: E731
        xm = synth.moe_token(seed, H)

        def moe_part(sel):
            return oracle.moe(st(lambda e: e.gate.codes, sel), st(lambda e: e.gate.scales, sel),
                              st(lambda e: e.up.codes, sel), st(lambda e: e.up.scales, sel),
                              st(lambda e: e.down.codes, sel), st(lambda e: e.down.scales, sel),
                              xm, np.arange(len(sel), dtype=np.int32), wts[list(sel)])

        one = _timed(lambda: moe_part(range(k)))
        parts = [list(range(k))[j::threads] for j in range(min(threads, k))]
        allc = _timed(lambda: np.sum(list(pool.map(moe_part, parts)), axis=0))
        b = roofline.moe_token_bytes(k, H, F)
        out["cfg5_moe_one_token_top16"] = {
            "one_thread_s": round(one, 4), "all_cores_s": round(allc, 4),
            "all_cores_threads": len(parts),
            "one_thread_GBs": round(b / one / 1e9, 4), "all_cores_GBs": round(b / allc / 1e9, 4),
            "algorithmic_bytes": int(b)}
        # cfg3
        shapes = synth.decode_step_shapes()
        step_w = sum(N * K for _, _, N, K in shapes)
        layer = [s for s in shapes if s[1].startswith("L0.")]
        layer_w = sum(N * K for _, _, N, K in layer)
        mats = [(synth.q4_matrix(seed, N, K, item=it), N, K) for it, _, N, K in layer]
        ext = {}
        for M in (16, 32):
            Xc = synth.activations(seed + 1, M, 4096)
            t1 = _timed(lambda: _split_rows(lambda a, c: oracle.q4_gemm(
                m.codes[a:c], m.scales[a:c], m.biases[a:c], Xc), 4096, threads, pool))
            tl = 0.0
            for mm, N, K in mats:
                X = synth.activations(seed + 1, M, K)
                tl += _timed(lambda: _split_rows(lambda a, c: oracle.q4_gemm(
                    mm.codes[a:c], mm.scales[a:c], mm.biases[a:c], X), N, threads, pool))
            tpass = tl * step_w / layer_w
            bpass = sum(roofline.q4_gemm_bytes(M, N, K) for _, _, N, K in shapes)
            ext["m%d" % M] = {
                "cfg1_matrix_all_cores_s": round(t1, 4), "layer_all_cores_s": round(tl, 4),
                "pass_all_cores_s_extrapolated": round(tpass, 3),
                "passes_per_s": round(1.0 / tpass, 6),
                "all_cores_GBs": round(bpass / tpass / 1e9, 4)}
        out["cfg3_verification_pass"] = dict(
            ext, kind="extrapolated", threads=threads,
            sample="one decoder layer (7 projections, %d weights) timed at M rows on %d threads, "
                   "scaled by the step's %d weights / the layer's (the lm_head included by that "
                   "ratio)" % (layer_w, threads, step_w))
    out["threads"] = threads
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed work before each measurement's warmup, so the "
                         "GPU clocks reach their sustained state")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-configs", action="store_true",
                    help="time the oracle on the decode step only (not configs 1, 3, 4, 5)")
    ap.add_argument("--no-m16", action="store_true", help="skip the verification passes")
    ap.add_argument("--verify-m", default="16,32",
                    help="activation rows of the timed verification passes (comma separated)")
    ap.add_argument("--no-per-shape", action="store_true",
                    help="skip timing each projection shape on its own")
    ap.add_argument("--no-kernel-compare", action="store_true",
                    help="skip timing both Q4 kernel families at M = 1, 2, 4")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the single-GEMV, int8 and MoE workloads")
    ap.add_argument("--traffic-pass", action="store_true",
                    help="run one decode step and one plain 1 GiB copy, for counter collection")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"))
    ap.add_argument("--counter-pass", metavar="MANIFEST_JSON",
                    help="launch every measured hot-path kernel once (and two calibration "
                         "kernels) for counter collection; write their algorithmic bytes")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "MANIFEST_JSON", "OUT_MD"))
    ap.add_argument("--summarize-sq", nargs="+", metavar="ARG",
                    help="MANIFEST_JSON OUT_MD CSV [CSV ...]: per-launch SQ/TCC counters")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV")
    ap.add_argument("--trace-csv", metavar="KERNEL_TRACE_CSV",
                    help="with --summarize-trace: the dispatch trace of the same run")
    ap.add_argument("--timed", nargs=2, type=int, metavar=("FIRST", "COUNT"),
                    help="with --trace-csv: the timed step launches, as bench.py reported them")
    ap.add_argument("--command", default="", help="command line recorded in summaries")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, command=args.command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, command=args.command)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq[2:], args.summarize_sq[0], args.summarize_sq[1],
                     command=args.command)
        return
    if args.counter_pass:
        counter_pass(args.counter_pass, args.seed)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command, args.trace_csv,
                        tuple(args.timed) if args.timed else None)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_weight_decode_dequant_amd as pkg
    from quantized_weight_decode_dequant_amd import _lib, roofline, synth, weights, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkg.raw()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log("device:", props.name, getattr(props, "gcnArchName", ""))

    t = time.time()
    step = workloads.build_decode_step(args.seed, log=log)
    log("workload ready in %.1f s: %d GEMVs, %.3f GB packed" % (
        time.time() - t, len(step.gemvs), step.weight_bytes / 1e9))
    step_bytes = step.algorithmic_bytes(1)

    # ---- decode step, M = 1: every GEMV of the step in one grouped launch
    Q4 = pkg.FMT_Q4_ASYM_G64
    plan = pkg.qg_batch_plan_build(Q4, 1, [(g.packed, g.N, g.K, g.x, g.y) for g in step.gemvs])
    torch.cuda.synchronize()
    log("plan: grid %d workgroups" % plan.grid)
    if args.traffic_pass:
        pkg.qg_batch_run(plan)
        torch.cuda.synchronize()
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("traffic pass: one decode step, one %d-byte copy" % COPY_BYTES)
        return
    # clocks settle first (the GPU runs a fresh workload below its sustained
    # clock for roughly the first 0.2 s), then the W warmup steps
    n_settle = workloads.settle(lambda: pkg.qg_batch_run(plan), args.settle)
    for _ in range(args.warmup):
        pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    # step-kernel launches so far: the graph check below adds none
    timed_first = n_settle + args.warmup
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        pkg.qg_batch_run(plan)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    log("step: %.3f ms (wall %.3f ms)" % (ms_step, wall * 1e3 / args.steps))
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    # one launch per step: the kernel's mean launch duration is the step time
    achieved = gbs
    traffic = traffic_from_profiles("q4_gemv_step")

    # ---- spread: 200 more steps in 20 groups of 10, an event pair around
    # each group (an event pair around every single launch reads about 3%
    # below the kernel's duration in the kernel trace, so it is not used)
    n_grp, per_grp = 20, 10
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_grp + 1)]
    ev[0].record()
    for k in range(n_grp):
        for _ in range(per_grp):
            pkg.qg_batch_run(plan)
        ev[k + 1].record()
    torch.cuda.synchronize()
    grp = np.array([ev[k].elapsed_time(ev[k + 1]) / per_grp for k in range(n_grp)])
    p10, p50, p90 = (float(np.percentile(grp, q)) for q in (10, 50, 90))
    log("step spread (%d groups of %d): p10 %.4f, median %.4f, p90 %.4f ms" % (
        n_grp, per_grp, p10, p50, p90))
    del ev

    # ---- the plain-read ceiling on this GPU, same run: best of a few grids
    rd = torch.empty(PLAIN_READ_BYTES, dtype=torch.uint8, device=dev)
    rd.fill_(1)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    plain_best, plain_grid = 0.0, 0
    for per_cu in (2, 4, 8, 16):
        grid = props.multi_processor_count * per_cu
        pkg.qg_plain_read(rd, sink, grid)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            pkg.qg_plain_read(rd, sink, grid)
        e1.record()
        torch.cuda.synchronize()
        r = PLAIN_READ_BYTES / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
        if r > plain_best:
            plain_best, plain_grid = r, grid
    log("plain read: %.1f GB/s (grid %d)" % (plain_best, plain_grid))
    del rd, sink

    # ---- for comparison: the same step as one qgemv_run launch per GEMV (HIP graph)
    graph = workloads.capture_graph(lambda: workloads.run_step_eager(step))
    graph.replay()
    torch.cuda.synchronize()
    n_cmp = max(3, args.steps // 5)
    e0.record()
    for _ in range(n_cmp):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_per_launch_graph = e0.elapsed_time(e1) / n_cmp
    log("step as %d launches in a graph: %.3f ms" % (len(step.gemvs), ms_per_launch_graph))
    del graph

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "synthetic dense decode step, M=1: 36 layers x (q 4096x4096, k/v 4096x1024, "
                        "o 4096x4096, gate/up 4096x12288, down 12288x4096) + lm_head 4096x151936, "
                        "4-bit asymmetric group-64, bf16 activations",
            "gemvs": len(step.gemvs),
            "packed_weight_bytes": step.weight_bytes,
            "algorithmic_bytes_per_step": int(step_bytes),
            "seed": args.seed,
            "launch": "one grouped kernel launch per step (qg_batch_run over a device work list "
                      "of the %d GEMVs)" % len(step.gemvs),
            "ms_per_step_one_launch_per_gemv": round(ms_per_launch_graph, 4),
            "timed_launches": [timed_first, args.steps],
        },
        "pct_of_peak": round(100 * gbs / roofline.HBM_PEAK_GBS, 2),
        "pct_of_plain_read": round(100 * gbs / plain_best, 2),
        "plain_read": {"value": round(plain_best, 1), "unit": "GB/s", "bytes": PLAIN_READ_BYTES,
                       "grid": plain_grid,
                       "kernel": "qg_plain_read: one contiguous share per workgroup, "
                                 "non-temporal 16-byte loads"},
        "ms_per_step_spread": {"steps": n_grp * per_grp, "groups_of": per_grp,
                               "p10": round(p10, 4), "median": round(p50, 4), "p90": round(p90, 4)},
        "tok_per_s": round(1e3 / ms_step, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "q4_gemv_kernel (work-list mode, one launch = one decode step)",
            "achieved": round(achieved, 2),
            "peak": roofline.HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / roofline.HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(step_bytes),
            "mean_launch_ms": round(ms_step, 5),
        },
    }

    # ---- verification passes: M-row activation tiles against the same
    # weights, one grouped launch per pass
    def time_pass(M, kernel=pkg.KERNEL_AUTO):
        Xs = [workloads.verification_tile(args.seed, g, M) for g in step.gemvs]
        Ys = [torch.empty((M, g.N), dtype=torch.bfloat16, device=dev) for g in step.gemvs]
        planM = pkg.qg_batch_plan_build(
            Q4, M, [(g.packed, g.N, g.K, X, Y) for g, X, Y in zip(step.gemvs, Xs, Ys)],
            kernel=kernel)
        workloads.settle(lambda: pkg.qg_batch_run(planM), args.settle)
        for _ in range(max(1, args.warmup)):
            pkg.qg_batch_run(planM)
        torch.cuda.synchronize()
        nM = max(5, args.steps // 2)
        e0.record()
        for _ in range(nM):
            pkg.qg_batch_run(planM)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nM, planM.plan.kernel

    if not args.no_m16:
        for M in [int(v) for v in args.verify_m.split(",") if v]:
            msM, _ = time_pass(M)
            bM = step.algorithmic_bytes(M)
            passes = 1e3 / msM
            result["m%d" % M] = {
                "ms_per_pass": round(msM, 4),
                "value": round(bM / (msM * 1e-3) / 1e9, 2),
                "unit": "GB/s",
                "pct_of_peak": round(100 * bM / (msM * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 2),
                "passes_per_s": round(passes, 2),
                # tokens per pass: 1 (no draft accepted), the pages' mean
                # accepted draft length, and M (every row accepted: the bound)
                "tok_per_s_equiv": {"tau_1": round(passes, 1),
                                    "tau_%s" % roofline.MEAN_ACCEPTED_TOKENS: round(
                                        passes * roofline.MEAN_ACCEPTED_TOKENS, 1),
                                    "tau_%d" % M: round(passes * M, 1)},
                "tflops": round(step.flops(M) / (msM * 1e-3) / 1e12, 2),
                "launch": "one grouped kernel launch per pass (%d-row activation tile per "
                          "projection)" % M,
            }
            log("m%d pass: %.3f ms" % (M, msM))

    # ---- each distinct projection shape on its own, one call per matrix
    # (the step's copies of that shape back to back, so the weights stream
    # from HBM; the single lm_head repeats, and 350 MB of it exceeds the
    # 256 MB last-level cache), at M = 1 (qgemv_run) and in verification
    # tiles (qgemm_skinny_run)
    def plain_read_us(nbytes: int) -> float:
        """Time of qg_plain_read over nbytes, distinct copies back to back (at
        least 1 GB of them, beyond the last-level cache), best of 1, 2 and 4
        workgroups per CU: the floor for one call that reads that much."""
        nbytes = nbytes // 16 * 16
        copies = max(2, min(256, (1 << 30) // nbytes + 1))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        for buf in bufs:
            buf.fill_(1)
        sink = torch.empty(65536, dtype=torch.int32, device=dev)
        best = None
        for per_cu in (1, 2, 4):
            grid = props.multi_processor_count * per_cu
            it = [0]

            def call():
                pkg.qg_plain_read(bufs[it[0] % copies], sink, grid)
                it[0] += 1

            us = workloads.time_graph_ms(call, min(copies, 64)) * 1e3
            best = us if best is None else min(best, us)
        del bufs
        return best

    if not args.no_per_shape:
        shapes = {}
        for g in step.gemvs:
            shapes.setdefault((g.name.split(".")[-1], g.N, g.K), []).append(g)
        per_shape, floors = {}, {}
        for (name, N, K), gs in shapes.items():
            wbytes = int(roofline.q4_gemm_bytes(1, N, K))
            if wbytes not in floors:
                floors[wbytes] = plain_read_us(wbytes)
            row = {"N": N, "K": K, "matrices": len(gs),
                   "plain_read_us": round(floors[wbytes], 2)}
            for M in [1] + [int(v) for v in args.verify_m.split(",") if v]:
                X = workloads.verification_tile(args.seed, gs[0], M)
                Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                it = [0]

                def call():
                    g = gs[it[0] % len(gs)]
                    it[0] += 1
                    if M == 1:
                        pkg.qgemv_run(Q4, g.packed, N, K, X[0], Y[0])
                    else:
                        pkg.qgemm_skinny_run(Q4, g.packed, M, N, K, X, Y=Y)

                ms = workloads.time_graph_ms(call, max(len(gs), 8))
                b = roofline.q4_gemm_bytes(M, N, K)
                row["m%d" % M] = {"us": round(ms * 1e3, 2),
                                  "GBs": round(b / (ms * 1e-3) / 1e9, 1),
                                  "pct_of_peak": round(100 * b / (ms * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 1),
                                  "pct_of_plain_read": round(100 * floors[wbytes] / (ms * 1e3), 1)}
            per_shape[name] = row
            log("shape %s %dx%d: plain read %.1f us; %s" % (name, N, K, floors[wbytes], ", ".join(
                "m%s %.1f us" % (k[1:], v["us"]) for k, v in row.items() if k.startswith("m") and k != "matrices")))
        result["per_shape"] = dict(per_shape, workload="one qgemv_run (M=1) or qgemm_skinny_run "
                                   "(M rows) per call, captured in a HIP graph, bf16 output; "
                                   "plain_read_us: qg_plain_read of the same weight bytes, one call, "
                                   "the floor for a call that size (launch and ramp included)")

    # ---- the two Q4 kernel families on the same pass, for the rows where
    # both apply: the default choice follows these figures
    if not args.no_kernel_compare:
        cmp = {}
        for M in (1, 2, 4):
            valu, _ = time_pass(M, pkg.KERNEL_VALU)
            mfma, _ = time_pass(M, pkg.KERNEL_MFMA)
            g0 = step.gemvs[0]
            auto = pkg.qg_batch_plan_build(
                Q4, M, [(g0.packed, g0.N, g0.K, workloads.verification_tile(args.seed, g0, M),
                         torch.empty((M, g0.N), dtype=torch.bfloat16, device=dev))]).plan.kernel
            cmp["m%d" % M] = {"valu_ms": round(valu, 4), "mfma_ms": round(mfma, 4),
                              "default": "valu" if auto == pkg.KERNEL_VALU else "mfma"}
            log("kernels m%d: valu %.3f ms, mfma %.3f ms" % (M, valu, mfma))
        result["kernel_choice"] = dict(
            cmp, workload="the verification pass over every projection of the decode step, "
                          "forced onto each kernel family (bf16 output)")

    # ---- the other workloads of the hot path, each against its own bytes
    if not args.no_extras:
        # single 4096 x 4096 GEMV (qgemv_run), the 72 distinct q/o matrices of
        # the step back to back (680 MB, larger than the last-level cache)
        sq = [g for g in step.gemvs if g.N == 4096 and g.K == 4096]
        it_sq = [0]

        def one_gemv():
            g = sq[it_sq[0] % len(sq)]
            it_sq[0] += 1
            pkg.qgemv_run(Q4, g.packed, g.N, g.K, g.x, g.y)

        ms1 = workloads.time_graph_ms(one_gemv, len(sq))
        b1 = roofline.q4_gemm_bytes(1, 4096, 4096)
        fl1 = plain_read_us(int(b1))
        result["single_gemv"] = {
            "plain_read_us": round(fl1, 2), "pct_of_plain_read": round(100 * fl1 / (ms1 * 1e3), 1),
            "workload": "4-bit g64 GEMV 4096x4096, M=1, one qgemv_run launch each, %d distinct "
                        "matrices back to back (captured in a HIP graph)" % len(sq),
            "us_per_gemv": round(ms1 * 1e3, 3),
            "value": round(b1 / (ms1 * 1e-3) / 1e9, 2), "unit": "GB/s",
            "pct_of_peak": round(100 * b1 / (ms1 * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 2)}
        log("single gemv: %.2f us" % (ms1 * 1e3))

        # 8-bit symmetric group-32 verification, M = 16, both projection shapes
        i8 = {}
        for N, K in ((12288, 4096), (4096, 12288)):
            wl = workloads.Int8Verify(args.seed, N, K)
            msq = workloads.time_graph_ms(wl.quantize, 40)
            msg = workloads.time_graph_ms(wl.gemm, len(wl.packed))
            bq = roofline.hadamard_quant_bytes(16, K)
            bg = roofline.q8_gemm_bytes(16, N, K)
            flg = plain_read_us(int(bg))
            i8["%dx%d" % (K, N)] = {
                "gemm_plain_read_us": round(flg, 2),
                "gemm_pct_of_plain_read": round(100 * flg / (msg * 1e3), 1),
                "hadamard_quant_us": round(msq * 1e3, 3),
                "hadamard_quant_GBs": round(bq / (msq * 1e-3) / 1e9, 2),
                "gemm_us": round(msg * 1e3, 3),
                "gemm_GBs": round(bg / (msg * 1e-3) / 1e9, 2),
                "gemm_pct_of_peak": round(100 * bg / (msg * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 2)}
            log("int8 %dx%d: hadamard %.2f us, gemm %.2f us" % (K, N, msq * 1e3, msg * 1e3))
            del wl
        result["int8_verify"] = dict(i8, workload="8-bit sym g32 weights, M=16 activations "
                                     "(1 percent x20 outliers) rotated by randomized Hadamard-32 and "
                                     "quantized to int8; %d copies of each matrix; calls captured in a HIP graph" % 40)

        # weight-only int8 output head (one fp32 scale per row), M = 1
        NH, KH = 151936, 4096
        gq = torch.Generator(device="cuda")
        gq.manual_seed(args.seed)
        qcodes = torch.randint(-128, 128, (NH, KH), dtype=torch.int8, device="cuda", generator=gq)
        qscales = (torch.rand(NH, dtype=torch.float32, device="cuda", generator=gq) + 0.5) * 2.0 ** -10
        qpacked = _lib.qgemv_pack(_lib.FMT_Q8_ROW, NH, KH, qcodes, qscales)
        del qcodes, qscales
        qx = weights.to_device(synth.activations(args.seed, 1, KH)[0], "cuda")
        qy = torch.empty(NH, dtype=torch.bfloat16, device="cuda")
        msh = workloads.time_graph_ms(
            lambda: _lib.qgemv_run(_lib.FMT_Q8_ROW, qpacked, NH, KH, qx, y=qy), 16)
        bh = roofline.q8row_gemv_bytes(NH, KH)
        flh = plain_read_us(int(bh))
        result["int8_lm_head"] = {
            "workload": "weight-only int8 output head 4096->151936, one fp32 scale per row, "
                        "codes uniform over the int8 range, M=1; calls captured in a HIP graph",
            "us": round(msh * 1e3, 3), "plain_read_us": round(flh, 2),
            "pct_of_plain_read": round(100 * flh / (msh * 1e3), 1),
            "value": round(bh / (msh * 1e-3) / 1e9, 2), "unit": "GB/s",
            "pct_of_peak": round(100 * bh / (msh * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 2)}
        log("int8 lm_head: %.2f us" % (msh * 1e3))
        del qpacked

        # the affine family at every width, group 64, fp16 scales: one GEMV
        # 8192 -> 262144 per width (codes drawn on the device)
        NA, KA, GA = 262144, 8192, 64
        rows = []
        for bits in (2, 3, 4, 5, 6, 8):
            fa = _lib.affine_format(bits, GA)
            ga = torch.Generator(device="cuda")
            ga.manual_seed(args.seed + bits)
            acodes = torch.randint(0, 1 << bits, (NA, KA), dtype=torch.uint8, device="cuda",
                                   generator=ga)
            asc = ((torch.rand(NA, KA // GA, device="cuda", generator=ga) + 0.05) * 0.02 * 15 /
                   ((1 << bits) - 1)).half().view(torch.int16)
            abi = (torch.randn(NA, KA // GA, device="cuda", generator=ga) * 0.01).half().view(torch.int16)
            apacked = _lib.qgemv_pack(fa, NA, KA, acodes, asc, abi)
            del acodes, asc, abi
            ax = weights.to_device(synth.activations(args.seed, 1, KA)[0], "cuda")
            ay = torch.empty(NA, dtype=torch.bfloat16, device="cuda")
            msa = workloads.time_graph_ms(
                lambda: _lib.qgemv_run(fa, apacked, NA, KA, ax, y=ay), 8)
            ba = roofline.affine_gemv_bytes(bits, GA, NA, KA)
            fla = plain_read_us(int(ba))
            # the same matrix against a 16-row activation tile (verification form)
            aX = weights.to_device(synth.activations(args.seed, 16, KA), "cuda")
            aY = torch.empty(16, NA, dtype=torch.bfloat16, device="cuda")
            ms16 = workloads.time_graph_ms(
                lambda: _lib.qgemm_skinny_run(fa, apacked, 16, NA, KA, aX, Y=aY), 8)
            b16 = roofline.affine_gemv_bytes(bits, GA, NA, KA) + 2.0 * 16 * KA + 2.0 * 16 * NA - 2.0 * KA - 2.0 * NA
            fl16 = fla * b16 / ba  # the same plain-read rate over the 16-row call's bytes
            rows.append({"bits": bits, "us": round(msa * 1e3, 2), "GBs": round(ba / (msa * 1e-3) / 1e9, 1),
                         "pct_of_peak": round(100 * ba / (msa * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 1),
                         "pct_of_plain_read": round(100 * fla / (msa * 1e3), 1),
                         "m16_us": round(ms16 * 1e3, 2),
                         "m16_GBs": round(b16 / (ms16 * 1e-3) / 1e9, 1),
                         "m16_pct_of_plain_read": round(100 * fl16 / (ms16 * 1e3), 1)})
            log("affine %d-bit g%d: %.2f us, M=16 %.2f us" % (bits, GA, msa * 1e3, ms16 * 1e3))
            del apacked, aX, aY
        result["affine_family"] = {
            "workload": "affine weights (scale * code + bias per group of 64, fp16), one GEMV "
                        "8192->262144 per code width, codes uniform, M=1, and the same matrix "
                        "against a 16-row bf16 tile (m16_*); calls captured in a HIP graph",
            "rows": rows}

        # the decode step's 253 projection shapes as 4-bit affine weights (group
        # 64, fp16; the Q4 step's bytes), all in one grouped launch
        fs = _lib.affine_format(4, GA)
        gs = torch.Generator(device="cuda")
        gs.manual_seed(args.seed + 100)
        sentries, bs = [], 0.0
        for item, name, N, K in synth.decode_step_shapes():
            scodes = torch.randint(0, 16, (N, K), dtype=torch.uint8, device="cuda", generator=gs)
            ssc = ((torch.rand(N, K // GA, device="cuda", generator=gs) + 0.05) * 0.02).half().view(torch.int16)
            sbi = (torch.randn(N, K // GA, device="cuda", generator=gs) * 0.01).half().view(torch.int16)
            sp = _lib.qgemv_pack(fs, N, K, scodes, ssc, sbi)
            del scodes, ssc, sbi
            sx = torch.randn(K, device="cuda", generator=gs).to(torch.bfloat16)
            sentries.append((sp, N, K, sx, torch.empty(N, dtype=torch.bfloat16, device="cuda")))
            bs += roofline.affine_gemv_bytes(4, GA, N, K)
        splan = _lib.qg_batch_plan_build(fs, 1, sentries)
        mss = workloads.time_graph_ms(lambda: _lib.qg_batch_run(splan), 20)
        result["affine_family"]["step_one_launch"] = {
            "workload": "the decode step's 253 projection shapes (36 layers of q, k, v, o, gate, "
                        "up, down and the 4096->151936 head) as 4-bit affine weights, group 64, "
                        "fp16 scale and bias, one seeded x each, M=1, one grouped launch per step "
                        "captured in a HIP graph",
            "ms": round(mss, 4), "GBs": round(bs / (mss * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * bs / (mss * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 1),
            "pct_of_plain_read": round(100 * bs / (mss * 1e-3) / 1e9 / plain_best, 1)}
        log("affine 4-bit decode step, one launch: %.4f ms" % mss)
        # the same weights against a 16-row activation tile per projection:
        # the verification pass in one grouped launch
        M16 = 16
        mentries, bm16 = [], 0.0
        for (sp, N, K, sx, sy) in sentries:
            mX = torch.randn(M16, K, device="cuda", generator=gs).to(torch.bfloat16)
            mentries.append((sp, N, K, mX, torch.empty((M16, N), dtype=torch.bfloat16,
                                                       device="cuda")))
            bm16 += roofline.affine_gemv_bytes(4, GA, N, K) + 2.0 * (M16 - 1) * (K + N)
        mplan = _lib.qg_batch_plan_build(fs, M16, mentries)
        msm16 = workloads.time_graph_ms(lambda: _lib.qg_batch_run(mplan), 20)
        result["affine_family"]["step_one_launch_m16"] = {
            "workload": "the same 253 affine products against a 16-row bf16 tile each (the "
                        "verification pass), one grouped launch captured in a HIP graph",
            "ms": round(msm16, 4), "GBs": round(bm16 / (msm16 * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * bm16 / (msm16 * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 1),
            "pct_of_plain_read": round(100 * bm16 / (msm16 * 1e-3) / 1e9 / plain_best, 1)}
        log("affine 4-bit verification pass M=16, one launch: %.4f ms" % msm16)
        del splan, sentries, mplan, mentries

        # the decode step's 253 shapes as weight-only int8 with row scales
        # (7.57 GB), all in one grouped launch
        gi = torch.Generator(device="cuda")
        gi.manual_seed(args.seed + 200)
        ientries, bi8 = [], 0.0
        for item, name, N, K in synth.decode_step_shapes():
            icodes = torch.randint(-128, 128, (N, K), dtype=torch.int8, device="cuda", generator=gi)
            isc = (torch.rand(N, dtype=torch.float32, device="cuda", generator=gi) + 0.5) * 2.0 ** -10
            ip = _lib.qgemv_pack(_lib.FMT_Q8_ROW, N, K, icodes, isc)
            del icodes, isc
            ix = torch.randn(K, device="cuda", generator=gi).to(torch.bfloat16)
            ientries.append((ip, N, K, ix, torch.empty(N, dtype=torch.bfloat16, device="cuda")))
            bi8 += roofline.q8row_gemv_bytes(N, K)
        iplan = _lib.qg_batch_plan_build(_lib.FMT_Q8_ROW, 1, ientries)
        msi = workloads.time_graph_ms(lambda: _lib.qg_batch_run(iplan), 10)
        result["int8_step_one_launch"] = {
            "workload": "the decode step's 253 projection shapes as weight-only int8 (one fp32 "
                        "scale per row, codes uniform over the int8 range), one seeded x each, "
                        "M=1, one grouped launch per step captured in a HIP graph",
            "ms": round(msi, 4), "GBs": round(bi8 / (msi * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * bi8 / (msi * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 1),
            "pct_of_plain_read": round(100 * bi8 / (msi * 1e-3) / 1e9 / plain_best, 1)}
        log("int8 decode step, one launch: %.4f ms" % msi)
        del iplan, ientries

        # MXFP4 routed experts, one token through one layer
        moe = workloads.MoeLayer(args.seed, 384, 7168, 2048, 16)
        msm = workloads.time_graph_ms(moe.run, 64)
        bm = roofline.moe_token_bytes(16, 7168, 2048)
        flm = plain_read_us(int(bm))
        result["moe"] = {
            "plain_read_us": round(flm, 2), "pct_of_plain_read": round(100 * flm / (msm * 1e3), 1),
            "workload": "MXFP4 MoE layer, 384 experts, hidden 7168, expert FFN 2048, top-16 "
                        "(a different seeded route per call), M=1; calls captured in a HIP graph",
            "us_per_token_layer": round(msm * 1e3, 3),
            "value": round(bm / (msm * 1e-3) / 1e9, 2), "unit": "GB/s",
            "pct_of_peak": round(100 * bm / (msm * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 2)}
        log("moe: %.2f us" % (msm * 1e3))
        del moe

        # the same layer for a verification tile: T positions, each its own route
        T = 16
        moet = workloads.MoeLayer(args.seed, 384, 7168, 2048, 16, T=T)
        mst = workloads.time_graph_ms(moet.run, 32)
        dist = moet.distinct_experts()
        bt = roofline.moe_positions_bytes(dist, T, 16, 7168, 2048)
        flt = plain_read_us(int(bt))
        result["moe_positions"] = {
            "workload": "MXFP4 MoE layer as above, %d positions per call, each with its own "
                        "seeded top-16 route (a different set per call); calls captured in a "
                        "HIP graph" % T,
            "T": T, "distinct_experts_mean": round(dist, 1),
            "us_per_pass": round(mst * 1e3, 3),
            "us_per_position": round(mst * 1e3 / T, 3),
            "vs_single_token_calls": round(T * msm / mst, 2),
            "plain_read_us": round(flt, 2), "pct_of_plain_read": round(100 * flt / (mst * 1e3), 1),
            "value": round(bt / (mst * 1e-3) / 1e9, 2), "unit": "GB/s",
            "pct_of_peak": round(100 * bt / (mst * 1e-3) / 1e9 / roofline.HBM_PEAK_GBS, 2)}
        log("moe T=%d: %.2f us (%.1f distinct experts)" % (T, mst * 1e3, dist))
        del moet

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(step, args.cpu_budget)
        threads = max(1, min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "16")), 16))
        result["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(step, args.cpu_budget / 2,
                                                                     threads)
        result["cpu_baseline"]["host"] = host_cpu_model()
        if not args.no_cpu_configs:
            t = time.time()
            result["cpu_baseline"]["configs"] = cpu_baseline_configs(args.seed, threads)
            log("cpu baseline, other configs: %.1f s" % (time.time() - t))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
