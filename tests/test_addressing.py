"""The scan kernels' buffer addressing, checked on the host: every load and
store of every tile, wave, lane and step over a sweep of ragged shapes lies
inside its tensor (the clamps in scan_linear_rnn_amd/csrc/scan_addr.hpp,
which the kernels call).  The same check built with a planted mistake (an
unclamped row offset in the forward scan) must report a violation."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "addr_check.cpp")
CSRC = os.path.join(ROOT, "scan_linear_rnn_amd", "csrc")


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def _build_and_run(tmp_path, *defines):
    exe = tmp_path / ("addr_check" + "".join(d.lower() for d in defines))
    cmd = [_hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{CSRC}",
           *(f"-D{d}" for d in defines), SRC, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)


def test_every_access_inside_its_tensor(tmp_path):
    res = _build_and_run(tmp_path)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("ok")


def test_check_reports_unclamped_rows(tmp_path):
    res = _build_and_run(tmp_path, "PLANT_UNCLAMPED_ROWS")
    assert res.returncode == 1
    assert "VIOLATION forward load" in res.stdout
