"""The C ABI: the shared library loads, exports every function the header
declares, sizes workspaces, and rejects bad arguments before launching
anything (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scanrnn.h")

sr = pytest.importorskip("scan_linear_rnn_amd")
lib = sr.raw_library()

FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_expected_calls():
    names = set(declared_functions())
    assert names == set(sr.EXPORTED), names


@pytest.mark.parametrize("name", declared_functions())
def test_every_declared_symbol_is_exported(name):
    assert hasattr(lib, name), name
    assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_empty_error():
    assert lib.scanrnn_version().decode().count(".") == 2
    assert isinstance(lib.scanrnn_last_error(), bytes)


def test_workspace_sizes():
    # Scan-only forward needs only the look-back words.  Large problems fuse
    # the input projection into the scan (look-back words of 128-step tiles,
    # no [k|p] staging); small ones stage [k|p].  W_out adds the h staging.
    s0 = lib.mingru_forward_workspace_size(8, 65536, 0, 1024, 1024, 0, 0)
    s1 = lib.mingru_forward_workspace_size(8, 65536, 1024, 1024, 1024, 1, 0)
    s2 = lib.mingru_forward_workspace_size(8, 65536, 1024, 1024, 1024, 1, 1)
    assert 0 < s0 < 2 ** 27
    assert 0 < s1 < 2 ** 27
    assert s1 >= 256 + 256 * 8 * 1024 * 8          # ceil(65536 / 256) tiles of words
    assert s2 - s1 >= 8 * 65536 * 1024 * 4
    small = lib.mingru_forward_workspace_size(2, 1024, 512, 512, 512, 1, 0)   # 128 tiles: staged
    assert small >= 2 * 1024 * 1024 * 4
    assert all(v % 256 == 0 for v in (s0, s1, s2, small))
    assert lib.minmax_scan_workspace_size(8, 32768, 192) > 0
    assert lib.mingru_forward_workspace_size(-1, 4, 4, 4, 4, 0, 0) == 0
    # The single-token step splits K inside the workgroup up to 512 streams
    # (no workspace); larger batches with K > 1024 split it across
    # workgroups, whose partial sums need workspace; tiny shapes need none.
    assert lib.mingru_step_workspace_size(256, 2048, 2048, 2048) == 0
    assert lib.mingru_step_workspace_size(512, 2048, 2048, 2048) == 0
    assert lib.mingru_step_workspace_size(1024, 2048, 2048, 2048) >= 1024 * 4096 * 4 * 2
    assert lib.mingru_step_workspace_size(2, 4, 4, 4) == 0


def test_workspace_sizes_with_zero_and_small_dims():
    """Every size query over grids that include zero dimensions (no input
    features, no state, no output, empty batch or sequence) returns without
    faulting, and K = 0 never asks for split-K partial sums."""
    import itertools
    for B, T, D_in, D_h, D_out in itertools.product([0, 1, 4, 600], [0, 1, 1000], [0, 1, 700],
                                                    [0, 1, 256], [0, 5]):
        for w_in, w_out in itertools.product([0, 1], [0, 1]):
            n = lib.mingru_forward_workspace_size(B, T, D_in, D_h, D_out, w_in, w_out)
            assert n % 256 == 0
        assert lib.mingru_step_workspace_size(B, D_in, D_h, D_out) >= 0
        assert lib.minmax_scan_workspace_size(B, T, D_h) >= 0
        assert lib.mingru_scan_backward_workspace_size(B, T, D_h) >= 0
    # No input features: the input product has K = 0 and needs no partial
    # sums; up to 4096 rows with K <= 1024 the K range is split inside each
    # workgroup; with K = 2048 it is split across workgroups. D_out = 0
    # leaves no output product.
    assert lib.mingru_step_workspace_size(1024, 0, 512, 0) == 0
    assert lib.mingru_step_workspace_size(1024, 1024, 512, 0) == 0
    assert lib.mingru_step_workspace_size(1024, 2048, 512, 0) > 0
    assert lib.mingru_step_workspace_size(8192, 1024, 64, 0) > 0  # few 128-row tiles past 4096 rows
    plain = lib.mingru_forward_workspace_size(4, 1000, 0, 256, 256, 1, 0)
    staged = 4 * 1000 * 2 * 256 * 4   # the [k|p] staging alone
    assert staged <= plain < staged + (1 << 20)


def _fwd(**kw):
    args = dict(B=2, T=8, D_in=0, D_h=4, D_out=4, x=None, W_in=None, k=FAKE, p=FAKE2,
                ld_kp=4, kp_dtype=sr.SR_F32, h0=None, W_out=None, y=FAKE, h_last=None,
                ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.mingru_forward(args["B"], args["T"], args["D_in"], args["D_h"], args["D_out"],
                              args["x"], args["W_in"], args["k"], args["p"], args["ld_kp"],
                              args["kp_dtype"], args["h0"], args["W_out"], args["y"],
                              args["h_last"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(T=-3), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(y=None), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(k=None), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(ld_kp=3), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(kp_dtype=7), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(D_out=5), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(x=FAKE), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(W_in=FAKE), sr.SR_ERR_INVALID_ARGUMENT),        # k, p must then be NULL
    (dict(y=ctypes.c_void_p(0x10002)), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(k=ctypes.c_void_p(0x10001), kp_dtype=1), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(ws=None), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(ws=ctypes.c_void_p(0x10040)), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=16), sr.SR_ERR_WORKSPACE_TOO_SMALL),
    (dict(B=1 << 40, T=1 << 40), sr.SR_ERR_INVALID_ARGUMENT),
])
def test_forward_rejects_bad_arguments(kw, code):
    assert _fwd(**kw) == code
    assert lib.scanrnn_last_error()


def test_oversized_later_launch_is_rejected_before_any_launch():
    """A scan-only forward whose scan fits one launch but whose output
    product's grid does not: the status is SR_ERR_UNSUPPORTED from the check
    pass, before the scan is enqueued (on this GPU-less host an attempted
    launch would report SR_ERR_HIP instead)."""
    B, T, D_h, D_out = 1, 262144, 1, 1 << 20
    st = _fwd(B=B, T=T, D_in=0, D_h=D_h, D_out=D_out, k=FAKE, p=FAKE2, ld_kp=1,
              W_out=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 40)
    assert st == sr.SR_ERR_UNSUPPORTED, lib.scanrnn_last_error()
    assert b"tiles too large" in lib.scanrnn_last_error()


def test_step_rejects_bad_arguments():
    f = lib.mingru_step
    need = lib.mingru_step_workspace_size(1024, 2048, 2048, 2048)  # K split across workgroups
    assert need > 0
    assert f(1024, 2048, 2048, 2048, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0,
             None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(1024, 2048, 2048, 2048, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need - 1,
             None) == sr.SR_ERR_WORKSPACE_TOO_SMALL
    assert f(-1, 4, 4, 4, FAKE, FAKE, None, None, FAKE, None, None, 0, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 4, 4, 4, FAKE, None, None, None, FAKE, None, None, 0, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 4, 4, 3, FAKE, FAKE, None, None, FAKE, None, None, 0, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 4, 4, 3, FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 4, 4, 4, FAKE, FAKE, None, None, None, None, None, 0, None) == sr.SR_ERR_INVALID_ARGUMENT


def test_minmax_rejects_bad_arguments():
    f = lib.minmax_scan
    big = 1 << 30
    assert f(2, 8, 4, FAKE, FAKE, None, FAKE, None, FAKE, big, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 8, 4, None, FAKE, FAKE, FAKE, None, FAKE, big, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 8, -4, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(2, 8, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, None) == sr.SR_ERR_WORKSPACE_TOO_SMALL
    assert f(2, 8, 4, FAKE, FAKE, FAKE, FAKE, None, None, big, None) == sr.SR_ERR_INVALID_ARGUMENT


def test_spin_limit_setter_bounds():
    text = open(HEADER).read()
    assert "#define SCANRNN_LOOKBACK_SPIN_LIMIT (1u << 20)" in text
    assert sr.LOOKBACK_SPIN_LIMIT == 1 << 20
    assert lib.scanrnn_set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT + 1) == sr.SR_ERR_INVALID_ARGUMENT
    assert b"above the default" in lib.scanrnn_last_error()
    assert lib.scanrnn_set_lookback_spin_limit(0) == sr.SR_OK
    assert lib.scanrnn_set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT) == sr.SR_OK
    with pytest.raises(ValueError):
        sr.set_lookback_spin_limit(-1)


def test_decayed_backward_rejects_bad_arguments():
    f = lib.mingru_scan_backward_decayed
    big = 1 << 30

    def call(**kw):
        a = dict(rate=FAKE, gap=FAKE, log1p=0, k=FAKE, p=FAKE2, ws=FAKE)
        a.update(kw)
        return f(2, 8, 4, a["k"], a["p"], 4, sr.SR_F32, a["rate"], a["gap"], a["log1p"], None,
                 FAKE, FAKE, None, FAKE, FAKE, None, a["ws"], big, None)
    assert call(rate=None) == sr.SR_ERR_INVALID_ARGUMENT
    assert b"decay_rate" in lib.scanrnn_last_error()
    assert call(gap=None) == sr.SR_ERR_INVALID_ARGUMENT
    assert call(log1p=2) == sr.SR_ERR_INVALID_ARGUMENT
    assert call(rate=ctypes.c_void_p(0x10002)) == sr.SR_ERR_INVALID_ARGUMENT
    assert call(ws=None) == sr.SR_ERR_INVALID_ARGUMENT


def test_status_requires_workspace():
    assert lib.scanrnn_workspace_status(None, None) == sr.SR_ERR_INVALID_ARGUMENT


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(2, 8, 4)
    with pytest.raises(ValueError):
        sr.minmax_scan(x, x, torch.zeros(2, 4))
    with pytest.raises((ValueError, TypeError)):
        sr.mingru_forward(k=x, p=x)


def _fwd_decayed(**kw):
    args = dict(B=2, T=8, D_in=0, D_h=4, D_out=4, x=None, W_in=None, k=FAKE, p=FAKE2,
                ld_kp=4, kp_dtype=sr.SR_F32, rate=FAKE, gap=FAKE2, log1p=0, sat=None,
                h0=None, W_out=None, y=FAKE, h_last=None, ws=FAKE, ws_bytes=16, stream=None)
    args.update(kw)
    return lib.mingru_forward_decayed(
        args["B"], args["T"], args["D_in"], args["D_h"], args["D_out"], args["x"], args["W_in"],
        args["k"], args["p"], args["ld_kp"], args["kp_dtype"], args["rate"], args["gap"],
        args["log1p"], args["sat"], args["h0"], args["W_out"], args["y"], args["h_last"],
        args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(rate=None), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(gap=None), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(log1p=2), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(rate=ctypes.c_void_p(0x10002)), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(sat=ctypes.c_void_p(0x10003)), sr.SR_ERR_INVALID_ARGUMENT),
    (dict(k=None), sr.SR_ERR_INVALID_ARGUMENT),          # the undecayed checks still apply
    (dict(), sr.SR_ERR_WORKSPACE_TOO_SMALL),             # valid decay arguments: reaches sizing
])
def test_forward_decayed_rejects_bad_arguments(kw, code):
    assert _fwd_decayed(**kw) == code
    assert lib.scanrnn_last_error()


def test_step_decayed_rejects_bad_arguments():
    f = lib.mingru_step_decayed
    need = lib.mingru_step_workspace_size(1024, 2048, 2048, 2048)
    args = [1024, 2048, 2048, 2048, FAKE, FAKE, FAKE]
    tail = [FAKE, FAKE, FAKE, FAKE, need - 1, None]   # h_prev, h_next, y_t, ws, bytes, stream
    assert f(*args, None, FAKE, 0, None, *tail) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(*args, FAKE, None, 0, None, *tail) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(*args, FAKE, FAKE, 5, None, *tail) == sr.SR_ERR_INVALID_ARGUMENT
    assert f(*args, FAKE, FAKE, 1, None, *tail) == sr.SR_ERR_WORKSPACE_TOO_SMALL


def test_header_is_plain_c_and_links(tmp_path):
    """The header compiles as C11 and a C program linked against the library
    gets the documented validation errors (no GPU needed: nothing launches)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi_check.c"
    src.write_text(r'''
#include <stdio.h>
#include "scanrnn.h"
int main(void) {
  float* fake = (float*)0x10000;
  if (mingru_forward(-1, 4, 0, 4, 4, 0, 0, fake, fake, 4, SR_F32, 0, 0, fake, 0, fake, 1u << 20, 0)
      != SR_ERR_INVALID_ARGUMENT) return 1;
  if (scanrnn_last_error()[0] == '\0') return 2;
  if (minmax_scan(2, 8, 4, fake, fake, 0, fake, 0, fake, 1u << 20, 0) != SR_ERR_INVALID_ARGUMENT)
    return 3;
  if (mingru_forward_workspace_size(8, 65536, 0, 1024, 1024, 0, 0) == 0) return 4;
  printf("%s\n", scanrnn_version());
  return 0;
}
''')
    lib = sr.library_path()
    exe = tmp_path / "abi_check"
    subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), lib, f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == lib_version()


def lib_version():
    return lib.scanrnn_version().decode()


def test_no_alloc_scan_validates_before_any_hip_call():
    """mingru_scan_noalloc refuses bad sizes and requests beyond its device
    array before touching the GPU (so this runs without one)."""
    assert lib.mingru_scan_noalloc_max_workspace() == 32 << 20
    st = lib.mingru_scan_noalloc(8, 1 << 17, 1024, FAKE, FAKE2, 1024, sr.SR_BF16, None, FAKE,
                                 None, None)
    assert st == sr.SR_ERR_UNSUPPORTED
    assert b"no-alloc scratch" in lib.scanrnn_last_error()
    assert lib.mingru_scan_noalloc(-1, 4, 4, FAKE, FAKE2, 4, sr.SR_F32, None, FAKE, None,
                                   None) == sr.SR_ERR_INVALID_ARGUMENT
    assert lib.mingru_scan_noalloc(2, 4, 8, FAKE, FAKE2, 4, sr.SR_F32, None, FAKE, None,
                                   None) == sr.SR_ERR_INVALID_ARGUMENT   # ld_kp < D
    assert lib.mingru_scan_noalloc(2, 4, 8, None, FAKE2, 8, sr.SR_F32, None, FAKE, None,
                                   None) == sr.SR_ERR_INVALID_ARGUMENT   # k missing
    assert lib.mingru_scan_noalloc(2, 4, 8, FAKE, FAKE2, 8, 7, None, FAKE, None,
                                   None) == sr.SR_ERR_INVALID_ARGUMENT   # dtype


def test_error_text_is_per_thread():
    """Each host thread sees its own last error: eight threads fail calls with
    different sizes at once (ctypes releases the GIL around each call) and
    every thread reads back the message of its own call."""
    import threading

    bad = {}

    def worker(i):
        for _ in range(300):
            st = lib.mingru_scan_noalloc(-(i + 1), 4, 4, FAKE, FAKE2, 4, sr.SR_F32, None, FAKE,
                                         None, None)
            msg = lib.scanrnn_last_error().decode()
            if st != sr.SR_ERR_INVALID_ARGUMENT or f"B={-(i + 1)} " not in msg:
                bad[i] = (st, msg)
                return

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad
