"""The library's calls under HIP graph capture: a token loop of mingru_step, a
scan-only forward and whole layer forwards are captured once and replayed
several times, with eager
work and synchronisations between the replays, and every replay must equal
the eager result bit for bit (the calls reset their workspaces with kernels,
never with memset nodes)."""

import numpy as np
import pytest
import torch

from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _steps(xs, W_in, W_out, h0):
    h = h0
    y = None
    for x_t in xs:
        y, h = sr.mingru_step(x_t, W_in, W_out, h_prev=h)
    return y, h


@pytest.mark.parametrize("B", [2, 64])
def test_step_loop_graph_replays_match_eager(B):
    say(f"graph step loop B={B}")
    rng = np.random.default_rng([1700, B])
    D, T = 256, 32
    W_in = dev((rng.standard_normal((D, 2 * D)) / D ** 0.5).astype(np.float32))
    W_out = dev((rng.standard_normal((D, D)) / D ** 0.5).astype(np.float32))
    xs = [dev(rng.standard_normal((B, D)).astype(np.float32)) for _ in range(T)]
    h0 = dev(rng.standard_normal((B, D)).astype(np.float32))
    y_ref, h_ref = _steps(xs, W_in, W_out, h0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        _steps(xs, W_in, W_out, h0)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_g, h_g = _steps(xs, W_in, W_out, h0)
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        y_g.zero_(); h_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h_g, h_ref) and torch.equal(y_g, y_ref), rep
        del junk


def test_scan_forward_graph_replays_match_eager():
    say("graph scan forward")
    rng = np.random.default_rng(1701)
    B, T, D = 4, 5000, 256
    k = dev(rng.normal(-2.0, 1.0, (B, T, D)).astype(np.float32))
    p = dev(rng.standard_normal((B, T, D)).astype(np.float32))
    h0 = dev(rng.standard_normal((B, D)).astype(np.float32))
    ref, ref_last = sr.mingru_forward(k=k, p=p, h0=h0, return_last=True)
    n = sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(ref)
    last = torch.empty_like(ref_last)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sr.mingru_forward(k=k, p=p, h0=h0, return_last=True, workspace=ws, out=out, out_last=last)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sr.mingru_forward(k=k, p=p, h0=h0, return_last=True, workspace=ws, out=out, out_last=last)
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        out.zero_(); last.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(last, ref_last), rep
        assert sr.workspace_status(ws) == 0
        del junk


@pytest.mark.parametrize("B,T,D_in,D_h,path", [
    (2, 1024, 512, 512, "narrow projections, reset, scan"),
    (8, 8192, 64, 1024, "projection fused with the scan, output projection"),
])
def test_layer_forward_graph_replays_match_eager(B, T, D_in, D_h, path):
    """The whole layer forward (x -> [k|p] -> scan -> y) captured once."""
    say(f"graph layer forward B={B} T={T} D_in={D_in} D_h={D_h}: {path}")
    rng = np.random.default_rng([1702, B, T])
    x = dev(rng.standard_normal((B, T, D_in)).astype(np.float32))
    W_in = dev((rng.standard_normal((D_in, 2 * D_h)) / D_in ** 0.5).astype(np.float32))
    W_out = dev((rng.standard_normal((D_h, D_in)) / D_h ** 0.5).astype(np.float32))
    h0 = dev(rng.standard_normal((B, D_h)).astype(np.float32))
    ref, ref_last = sr.mingru_forward(x, W_in, W_out=W_out, h0=h0, return_last=True)
    n = sr.raw_library().mingru_forward_workspace_size(B, T, D_in, D_h, D_in, 1, 1)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(ref)
    last = torch.empty_like(ref_last)

    def fwd():
        sr.mingru_forward(x, W_in, W_out=W_out, h0=h0, return_last=True, workspace=ws,
                          out=out, out_last=last)

    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        out.zero_(); last.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(last, ref_last), rep
        assert sr.workspace_status(ws) == 0
        del junk
