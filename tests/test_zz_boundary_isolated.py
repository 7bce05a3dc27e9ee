"""The C-ABI boundary tests (test_boundary.py) on a GPU host.

Those tests pass fake device addresses to calls that must fail validation
before any HIP call.  On a host with a GPU they run here, in a child process
with every GPU hidden, so that a regressed host check surfaces as a failed
assertion (the launch returns QG_EHIP) rather than as a GPU memory fault."""
import os
import subprocess
import sys

import pytest

from conftest import HIDE_GPUS, ROOT, gpu_visible


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_visible(), reason="no GPU: test_boundary.py runs directly")
def test_boundary_module_with_gpus_hidden():
    env = dict(os.environ, QG_BOUNDARY_CHILD="1", **HIDE_GPUS)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert " passed" in r.stdout and " skipped" not in r.stdout.split("\n")[-2], r.stdout[-500:]
