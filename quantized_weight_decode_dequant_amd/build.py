"""Ahead-of-time build of the HIP library for gfx950 (in-tree shared object)."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libqgemv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, flush=True)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source into libqgemv.so (always recompiles): one
    object per source, compiled in parallel, then one shared-object link."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="qgemv_build_") as d:
        objs = [os.path.join(d, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[HIPCC, *compile_flags, "-c", "-o", o, src] for src, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
