"""The allocation-free scan (mingru_scan_noalloc) through the C ABI: its
results equal mingru_forward's (scan-only, with a caller workspace) bit for
bit, on two calls in a row, the second smaller than the first (the shared
device array keeps the last call's contents, and each call resets what it
uses); a request beyond the array is refused and writes nothing."""

import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")
lib = sr.raw_library()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _inputs(B, T, D, dtype, seed, with_h0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    k = torch.empty((B, T, D), device="cuda").normal_(-3.0, 1.5, generator=g).to(dtype)
    p = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g).to(dtype)
    h0 = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g) if with_h0 else None
    return k, p, h0


def _with_workspace(k, p, h0):
    B, T, D = k.shape
    kd = sr.SR_BF16 if k.dtype == torch.bfloat16 else sr.SR_F32
    nb = lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    h = torch.empty((B, T, D), device="cuda")
    last = torch.empty((B, D), device="cuda")
    st = lib.mingru_forward(B, T, 0, D, D, None, None, _ptr(k), _ptr(p), D, kd, _ptr(h0), None,
                            _ptr(h), _ptr(last), _ptr(ws), nb, _stream())
    assert st == 0, lib.scanrnn_last_error()
    return h, last


def _no_alloc(k, p, h0):
    B, T, D = k.shape
    kd = sr.SR_BF16 if k.dtype == torch.bfloat16 else sr.SR_F32
    h = torch.full((B, T, D), float("nan"), device="cuda")
    last = torch.full((B, D), float("nan"), device="cuda")
    st = lib.mingru_scan_noalloc(B, T, D, _ptr(k), _ptr(p), D, kd, _ptr(h0), _ptr(h), _ptr(last),
                                 _stream())
    assert st == 0, lib.scanrnn_last_error()
    return h, last


def test_no_alloc_scan_equals_the_workspace_scan_twice_in_a_row():
    cases = [(8, 20000, 1024, torch.bfloat16, 1, True), (2, 3001, 200, torch.float32, 2, False)]
    for B, T, D, dtype, seed, with_h0 in cases:
        say(f"no-alloc scan B={B} T={T} D={D} {dtype} h0={with_h0}")
        k, p, h0 = _inputs(B, T, D, dtype, seed, with_h0)
        want, want_last = _with_workspace(k, p, h0)
        got, got_last = _no_alloc(k, p, h0)
        torch.cuda.synchronize()
        assert torch.equal(got, want) and torch.equal(got_last, want_last), (B, T, D)


def test_no_alloc_scan_refuses_requests_beyond_its_array():
    B, T, D = 8, 1 << 17, 1024          # needs more look-back words than 32 MiB hold
    say("no-alloc scan beyond the array")
    assert lib.mingru_scan_noalloc_max_workspace() == 32 << 20
    h = torch.full((2, 4), 7.0, device="cuda")
    st = lib.mingru_scan_noalloc(B, T, D, ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), D,
                                 sr.SR_BF16, None, _ptr(h), None, _stream())
    assert st == sr.SR_ERR_UNSUPPORTED
    assert b"no-alloc scratch" in lib.scanrnn_last_error()
    torch.cuda.synchronize()
    assert torch.all(h == 7.0)
