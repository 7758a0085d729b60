"""The library called from plain C (rejection_sampling_verify_13_amd/examples/
verify_from_c.c, built next to the library by the package build): the
two-token worked example of the zwjcode.cn page, section 05, through
spec_verify with device buffers from the HIP runtime, must commit [A] = [0, -1]
with no draft accepted, and spec_verify_device_errors must report no faulted
request."""
import os
import subprocess

import pytest

from parity import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "rejection_sampling_verify_13_amd", "verify_from_c")


def test_worked_example_from_c():
    if not os.path.exists(EXE):
        pytest.fail("verify_from_c is not built; run __graft_entry__.build()")
    log("[c] worked example through the C ABI")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    log("[c] %s" % r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "tokens [0, -1], accepted 0, faulted requests 0"
