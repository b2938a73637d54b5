"""GPU parity of the MinMax scan: bit for bit against the sequential oracle."""

import numpy as np
import pytest
import torch

import synth
from oracle import metrics, minmax
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _inputs(B, T, D, seed):
    rng = np.random.default_rng([600, seed])
    r = rng.uniform(-1, 1, (B, T, D)).astype(np.float32)
    s = (rng.uniform(-1, 1, (B, T, D)) - 0.5).astype(np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    for a in (r, s, x0):
        a[a == 0] = 0.0
    return r, s, x0


@pytest.mark.parametrize("B,T,D", [
    (2, 64, 16), (3, 1000, 200), (1, 1, 5), (2, 5000, 192), (4, 3333, 7), (1, 40000, 64),
    # 32 chains of one channel per lane: the 240-step tiles, ragged in T and D.
    (8, 5001, 200), (16, 241, 65),
])
def test_minmax_bitwise(B, T, D):
    say(f"minmax B={B} T={T} D={D}")
    r, s, x0 = _inputs(B, T, D, seed=B + T + D)
    out, last = sr.minmax_scan(dev(r), dev(s), dev(x0), return_last=True)
    ref, ref_last = minmax.scan(r, s, x0)
    assert metrics.bits_equal(out.cpu().numpy(), ref)
    assert metrics.bits_equal(last.cpu().numpy(), ref_last)


def test_minmax_full_size_b8_t32768_d192_bitwise():
    cfg = synth.CONFIGS[synth.MINMAX]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    say("minmax full size B=8 T=32768 D=192")
    r = synth.uniform_bt(synth.MINMAX, "r", B, T, D, -1.0, 1.0)
    s = synth.uniform_bt(synth.MINMAX, "s", B, T, D, -1.0, 1.0) - np.float32(0.5)
    s[s == 0] = 0.0
    x0 = synth.uniform_vec(synth.MINMAX, "x0", B, D, -1.0, 1.0)
    out, last = sr.minmax_scan(dev(r), dev(s), dev(x0), return_last=True)
    ref, ref_last = minmax.scan(r, s, x0)
    assert metrics.bits_equal(out.cpu().numpy(), ref)
    assert metrics.bits_equal(last.cpu().numpy(), ref_last)


def test_minmax_hold_and_single_reset_across_tiles():
    B, T, D = 2, 30000, 192
    rng = np.random.default_rng(601)
    r = np.full((B, T, D), 2.0, np.float32)
    s = np.full((B, T, D), -2.0, np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    out = sr.minmax_scan(dev(r), dev(s), dev(x0)).cpu().numpy()
    assert np.array_equal(out, np.broadcast_to(x0[:, None, :], out.shape))
    tstar = 17777
    v = rng.uniform(-1.5, 1.5, (B, D)).astype(np.float32)
    r[:, tstar] = -3.0
    s[:, tstar] = v
    out = sr.minmax_scan(dev(r), dev(s), dev(x0)).cpu().numpy()
    assert np.array_equal(out[:, :tstar], np.broadcast_to(x0[:, None, :], (B, tstar, D)))
    assert np.array_equal(out[:, tstar:], np.broadcast_to(v[:, None, :], (B, T - tstar, D)))


def test_minmax_repeated_and_split_calls_identical():
    B, T, D = 3, 9000, 192
    r, s, x0 = _inputs(B, T, D, seed=602)
    rd, sd, xd = dev(r), dev(s), dev(x0)
    full, last = sr.minmax_scan(rd, sd, xd, return_last=True)
    for _ in range(2):
        assert torch.equal(sr.minmax_scan(rd, sd, xd), full)
    T1 = 4321
    a, la = sr.minmax_scan(rd[:, :T1].contiguous(), sd[:, :T1].contiguous(), xd, return_last=True)
    b, lb = sr.minmax_scan(rd[:, T1:].contiguous(), sd[:, T1:].contiguous(), la, return_last=True)
    assert torch.equal(torch.cat([a, b], dim=1), full) and torch.equal(lb, last)


def test_minmax_empty_sequence():
    x0 = dev(np.float32([[0.5, -0.25]]))
    e = torch.zeros((1, 0, 2), device="cuda")
    out, last = sr.minmax_scan(e, e, x0, return_last=True)
    assert out.shape == (1, 0, 2) and torch.equal(last, x0)


def test_minmax_step_matches_scan_bitwise():
    """Token-by-token steps (streaming, one token per call) reproduce the
    parallel scan bit for bit, in place."""
    B, T, D = 3, 200, 192
    r, s, x0 = _inputs(B, T, D, seed=650)
    rd, sd = dev(r), dev(s)
    full = sr.minmax_scan(rd, sd, dev(x0))
    x = dev(x0).clone()
    for t in range(T):
        y = sr.minmax_step(rd[:, t].contiguous(), sd[:, t].contiguous(), x, x_next=x)
        assert y.data_ptr() == x.data_ptr()
        assert torch.equal(x, full[:, t])


def test_minmax_three_chains_long_sequence_bitwise():
    """B=1, T=2^18, D=192: three chains of ~910 tiles, all of them in flight
    together, so most tiles resolve through long look-back walks.  The
    forward bit for bit against the oracle; the backward's routing exactly,
    its routed values (fp32 sums of upstream gradients) within rounding."""
    from oracle import grad
    B, T, D = 1, 1 << 18, 192
    say(f"minmax three chains B={B} T={T} D={D}")
    r, s, x0 = _inputs(B, T, D, 31)
    rd, sd, x0d = dev(r), dev(s), dev(x0)
    out, last = sr.minmax_scan(rd, sd, x0d, return_last=True)
    ref, ref_last = minmax.scan(r, s, x0)
    assert metrics.bits_equal(out.cpu().numpy(), ref)
    assert metrics.bits_equal(last.cpu().numpy(), ref_last)
    rng = np.random.default_rng(632)
    dx = rng.standard_normal((B, T, D)).astype(np.float32)
    dr, ds, dx0 = sr.minmax_scan_backward(rd, sd, x0d, out, dev(dx))
    rdr, rds, rdx0 = grad.minmax_scan_backward(r, s, x0, dx)
    assert np.array_equal(dr.cpu().numpy() != 0, rdr != 0)
    assert np.array_equal(ds.cpu().numpy() != 0, rds != 0)
    scale = np.abs(dx).sum(axis=1).max()
    for got, want in ((dr, rdr), (ds, rds), (dx0, rdx0)):
        assert float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - want))) < 1e-5 * scale
