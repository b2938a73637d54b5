"""Every scan reads and writes only inside its tensors: inputs and outputs are
placed so that they end exactly at the end of their own device allocation
(hipMalloc, no caching allocator around them), with ragged shapes whose last
tile straddles the end of the sequence and of the channels.  The kernels
clamp their rows and lanes (scan_addr.hpp; checked access by access on the
host in test_addressing.py); these runs confirm it on the device, and compare
with the same calls on ordinary tensors, bit for bit."""

import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")
lib = sr.raw_library()

_D2D = 3  # hipMemcpyDeviceToDevice
_GRAIN = 2 << 20


class _EndPlaced:
    """A tensor's bytes placed at the very end of a fresh hipMalloc block."""

    def __init__(self, hip, t: torch.Tensor):
        self.hip = hip
        self.nbytes = t.numel() * t.element_size()
        self.size = max((self.nbytes + _GRAIN - 1) // _GRAIN * _GRAIN, _GRAIN)
        self.block = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(self.block), ctypes.c_size_t(self.size)) == 0
        self.ptr = ctypes.c_void_p(self.block.value + self.size - self.nbytes)
        torch.cuda.synchronize()
        assert hip.hipMemcpy(self.ptr, ctypes.c_void_p(t.data_ptr()), ctypes.c_size_t(self.nbytes),
                             _D2D) == 0

    def read_into(self, t: torch.Tensor):
        torch.cuda.synchronize()
        assert self.hip.hipMemcpy(ctypes.c_void_p(t.data_ptr()), self.ptr,
                                  ctypes.c_size_t(self.nbytes), _D2D) == 0
        return t

    def free(self):
        torch.cuda.synchronize()
        self.hip.hipFree(self.block)


@pytest.fixture(scope="module")
def hip():
    h = ctypes.CDLL("libamdhip64.so.7")
    h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    h.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    h.hipFree.argtypes = [ctypes.c_void_p]
    return h


def _ws(nbytes):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("B,T,D,dtype,halves", [
    (3, 1001, 200, torch.float32, False),   # one channel per lane, lanes past D, ragged T
    (2, 701, 130, torch.bfloat16, False),
    (40, 333, 130, torch.float32, False),   # two channels per lane (>= 32 chains)
    (2, 517, 96, torch.float32, True),      # k and p the halves of one [B,T,2D] buffer
])
def test_forward_scan_inputs_and_output_end_at_the_allocation(hip, B, T, D, dtype, halves):
    say(f"bounds: forward B={B} T={T} D={D} {dtype} halves={halves}")
    g = torch.Generator(device="cuda")
    g.manual_seed(2200 + T)
    if halves:
        kp = torch.empty((B, T, 2 * D), device="cuda").normal_(-1.0, 1.5, generator=g).to(dtype)
        k_ref, p_ref = kp[..., :D], kp[..., D:]
        buf = _EndPlaced(hip, kp)
        esz = kp.element_size()
        k_ptr, p_ptr, ld = buf.ptr, ctypes.c_void_p(buf.ptr.value + D * esz), 2 * D
        bufs = [buf]
    else:
        k_ref = torch.empty((B, T, D), device="cuda").normal_(-1.0, 1.5, generator=g).to(dtype)
        p_ref = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g).to(dtype)
        kb, pb = _EndPlaced(hip, k_ref), _EndPlaced(hip, p_ref)
        k_ptr, p_ptr, ld = kb.ptr, pb.ptr, D
        bufs = [kb, pb]
    h0 = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    want, want_last = sr.mingru_forward(k=k_ref, p=p_ref, h0=h0, return_last=True)
    y = _EndPlaced(hip, torch.empty_like(want))
    last = _EndPlaced(hip, torch.empty_like(want_last))
    bufs += [y, last]
    nb = lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0)
    ws = _ws(nb)
    kd = sr.SR_BF16 if dtype == torch.bfloat16 else sr.SR_F32
    st = lib.mingru_forward(B, T, 0, D, D, None, None, k_ptr, p_ptr, ld, kd,
                            ctypes.c_void_p(h0.data_ptr()), None, y.ptr, last.ptr,
                            ctypes.c_void_p(ws.data_ptr()), nb, _stream())
    assert st == 0, lib.scanrnn_last_error()
    got = y.read_into(torch.empty_like(want))
    got_last = last.read_into(torch.empty_like(want_last))
    for b in bufs:
        b.free()
    assert torch.equal(got, want) and torch.equal(got_last, want_last)


def test_minmax_scan_inputs_and_output_end_at_the_allocation(hip):
    B, T, D = 3, 1001, 200
    say(f"bounds: minmax B={B} T={T} D={D}")
    g = torch.Generator(device="cuda")
    g.manual_seed(2210)
    r = torch.empty((B, T, D), device="cuda").uniform_(-1, 1, generator=g)
    s = torch.empty((B, T, D), device="cuda").uniform_(-1.5, 0.5, generator=g)
    x0 = torch.empty((B, D), device="cuda").uniform_(-1, 1, generator=g)
    want = sr.minmax_scan(r, s, x0)
    rb, sb, ob = _EndPlaced(hip, r), _EndPlaced(hip, s), _EndPlaced(hip, torch.empty_like(want))
    nb = lib.minmax_scan_workspace_size(B, T, D)
    ws = _ws(nb)
    st = lib.minmax_scan(B, T, D, rb.ptr, sb.ptr, ctypes.c_void_p(x0.data_ptr()), ob.ptr, None,
                         ctypes.c_void_p(ws.data_ptr()), nb, _stream())
    assert st == 0, lib.scanrnn_last_error()
    got = ob.read_into(torch.empty_like(want))
    for b in (rb, sb, ob):
        b.free()
    assert torch.equal(got, want)


@pytest.mark.parametrize("B,T,D", [(3, 1001, 200), (40, 333, 130)])
def test_backward_scan_tensors_end_at_the_allocation(hip, B, T, D):
    say(f"bounds: backward B={B} T={T} D={D}")
    g = torch.Generator(device="cuda")
    g.manual_seed(2220 + T)
    k = torch.empty((B, T, D), device="cuda").normal_(-1.0, 1.5, generator=g)
    p = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    h0 = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    h = sr.mingru_forward(k=k, p=p, h0=h0)
    dh = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    want = sr.mingru_scan_backward(k, p, h, dh, h0=h0)
    ins = [_EndPlaced(hip, t) for t in (k, p, h, dh)]
    outs = [_EndPlaced(hip, torch.empty_like(t)) for t in want]
    nb = lib.mingru_scan_backward_workspace_size(B, T, D)
    ws = _ws(nb)
    st = lib.mingru_scan_backward(B, T, D, ins[0].ptr, ins[1].ptr, D, sr.SR_F32,
                                  ctypes.c_void_p(h0.data_ptr()), ins[2].ptr, ins[3].ptr, None,
                                  outs[0].ptr, outs[1].ptr, outs[2].ptr,
                                  ctypes.c_void_p(ws.data_ptr()), nb, _stream())
    assert st == 0, lib.scanrnn_last_error()
    got = [o.read_into(torch.empty_like(w)) for o, w in zip(outs, want)]
    for b in ins + outs:
        b.free()
    for a, b in zip(got, want):
        assert torch.equal(a, b)
