"""Builds libscanrnn.so (HIP, gfx950) in the package directory.

    python scan_linear_rnn_amd/build.py        # or __graft_entry__.build()

(Run it as a script: importing the package would load the library it builds.)

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
generation switched off (-packed-fp32-ops), and linked into one shared
library exporting the C ABI declared in include/scanrnn.h.

build_host_sanitized(out_dir) makes a second copy whose HOST code (argument
validation, sizing, launch set-up) is built with AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is the same as in the normal
build.  Load it with SCANRNN_LIBRARY=<path> and the ASan runtime preloaded
(host_sanitizer_env gives the environment); it is for CPU tests of the C ABI.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libscanrnn.so")

ARCH = "gfx950"
SOURCES = ["scan.hip", "scan_bwd.hip", "gemm.hip", "fused.hip", "noalloc.hip", "api.cpp"]
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *extra]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-only sanitizer flags: each -fsanitize= applies to the host pass only.
SANITIZE_HOST = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]


def asan_runtime() -> str:
    """The clang ASan runtime that a sanitized library needs preloaded."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "llvm")
    res = subprocess.run([os.path.join(llvm, "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"ASan runtime not found ({res.stdout.strip()} {res.stderr.strip()})")
    return path


def build_host_sanitized(out_dir: str) -> str:
    """Builds libscanrnn_hostsan.so in out_dir (see the module docstring)."""
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, SANITIZE_HOST), SOURCES))
    lib = os.path.join(out_dir, "libscanrnn_hostsan.so")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return lib


def host_sanitizer_env(lib: str, log_prefix: str | None = None) -> dict:
    """Environment for a Python process that loads the sanitized library:
    the ASan runtime first, leak checks off (the interpreter keeps its
    allocations), the first report fatal; reports also go to files
    log_prefix.<pid> when a prefix is given."""
    env = dict(os.environ)
    env["SCANRNN_LIBRARY"] = lib
    env["LD_PRELOAD"] = asan_runtime()
    log = f":log_path={log_prefix}" if log_prefix else ""
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0" + log
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1" + log
    return env


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
