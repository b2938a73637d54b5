"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
a copy of the library with sanitized host code (device code unchanged) runs
the CPU tests of the ABI (tests/test_abi.py: loading, symbol export, sizing,
every rejection path) in a child process; any sanitizer report fails it."""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_scanrnn_build", os.path.join(ROOT, "scan_linear_rnn_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    build = _build_module()
    try:
        build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_host_sanitized(str(tmp_path / "hostsan"))
    # The copy's host code calls the sanitizer runtimes (so the run below
    # really exercises instrumented validation code).
    with open(lib, "rb") as f:
        image = f.read()
    assert b"__asan_report_load8" in image and b"__ubsan_handle_" in image
    logs = tmp_path / "reports"
    logs.mkdir()
    env = build.host_sanitizer_env(lib, str(logs / "san"))
    # In the child, the binding reports which file it loaded; then the ABI
    # tests run (all but the one that links a C program against the library
    # with the system linker, which would need the sanitizer runtimes too).
    probe = subprocess.run(
        [sys.executable, "-c", "import scan_linear_rnn_amd as sr; print(sr.library_path())"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.split()[-1] == lib
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not plain_c_and_links"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    reports = "".join(open(p).read() for p in sorted(logs.iterdir()))
    assert not reports, reports[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert " passed" in out and "failed" not in out, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
