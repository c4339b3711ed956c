"""CPU check of the launch-epoch and tag arithmetic that keeps stale look-back
records from being read as current (csrc/tags.hpp): builds
tests/epoch_check.cpp as a host program against the library's own header and
runs it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nonlinear_rnn_solve_pararnn_amd", "csrc")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_epoch_arithmetic(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "epoch_check")
    src = os.path.join(ROOT, "tests", "epoch_check.cpp")
    r = subprocess.run([cc, "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
