"""Forced look-back time-outs.

The poll budget of the look-back's bounded wait is lowered from the host
(scanrnn_set_lookback_spin_limit(0): a tile gives up at the first
predecessor word it finds unwritten), so the give-up path runs while every
kernel still ends normally -- the waits only end sooner.  A tile that gives
up marks its workspace and carries NaN for that channel; every result it does
not reach keeps the bits of a normal run (the carry is the same fma sequence
whichever predecessor state it starts from); the default budget restores
normal results.  MinMax is covered by the status only: min and max drop a
NaN operand, so values after a give-up are wrong but finite.
"""

import pytest
import torch

import scan_linear_rnn_amd as sr
import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture
def zero_polls():
    sr.set_lookback_spin_limit(0)
    try:
        yield
    finally:
        sr.set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT)


def _ws(nbytes):
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda")


def _compare(name, outs, refs, status):
    """Give-ups are flagged exactly when some output is NaN, and the outputs
    they do not reach equal the normal run's bit for bit."""
    nan = any(bool(torch.isnan(o).any()) for o in outs)
    say(f"{name}: status {status}, NaN outputs {nan}")
    assert (status == sr.SR_ERR_LOOKBACK_TIMEOUT) == nan
    for o, r in zip(outs, refs):
        keep = ~torch.isnan(o)
        assert torch.equal(o[keep], r[keep])
    return status == sr.SR_ERR_LOOKBACK_TIMEOUT


def _scan_inputs():
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    k = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    p = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    return k, p, h0


def test_scan_and_backward_give_up_visibly_and_recover():
    """B=8, T=65536, D=1024 (bf16 k/p): ~3700 tiles with up to 512 in flight,
    so with no polls some tile meets an unwritten predecessor word."""
    say("forced time-outs: scan and backward B=8 T=65536 D=1024")
    k, p, h0 = _scan_inputs()
    B, T, D = k.shape
    lib = sr.raw_library()
    ws = _ws(lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0))
    ref, ref_last = sr.mingru_forward(k=k, p=p, h0=h0, return_last=True, workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    g = torch.Generator(device="cuda")
    g.manual_seed(1130)
    dh = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    wsb = _ws(lib.mingru_scan_backward_workspace_size(B, T, D))
    bref = sr.mingru_scan_backward(k, p, ref, dh, h0=h0, workspace=wsb)
    assert sr.workspace_status(wsb) == sr.SR_OK

    sr.set_lookback_spin_limit(0)
    try:
        out, last = sr.mingru_forward(k=k, p=p, h0=h0, return_last=True, workspace=ws)
        hit_f = _compare("forward", [out, last], [ref, ref_last], sr.workspace_status(ws))
        bout = sr.mingru_scan_backward(k, p, ref, dh, h0=h0, workspace=wsb)
        hit_b = _compare("backward", list(bout), list(bref), sr.workspace_status(wsb))
    finally:
        sr.set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT)
    assert hit_f and hit_b  # the budget reached the kernels

    out, last = sr.mingru_forward(k=k, p=p, h0=h0, return_last=True, workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    assert torch.equal(out, ref) and torch.equal(last, ref_last)
    bout = sr.mingru_scan_backward(k, p, ref, dh, h0=h0, workspace=wsb)
    assert sr.workspace_status(wsb) == sr.SR_OK
    assert all(torch.equal(a, b) for a, b in zip(bout, bref))


def test_fused_projection_scan_gives_up_visibly_and_recovers(zero_polls):
    """The projection fused with the scan (B=8, T=8192, D_in=64, D_h=1024:
    4096 tiles of 256 steps x 64 channels) runs the same look-back."""
    B, T, D_in, D_h = 8, 8192, 64, 1024
    say(f"forced time-outs: fused forward B={B} T={T} D_in={D_in} D_h={D_h}")
    g = torch.Generator(device="cuda")
    g.manual_seed(4401)
    x = torch.randn(B, T, D_in, device="cuda", generator=g)
    W = torch.randn(D_in, 2 * D_h, device="cuda", generator=g) / D_in ** 0.5
    h0 = torch.randn(B, D_h, device="cuda", generator=g)
    ws = _ws(sr.raw_library().mingru_forward_workspace_size(B, T, D_in, D_h, D_h, 1, 0))
    sr.set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT)
    ref = sr.mingru_forward(x, W, h0=h0, workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    sr.set_lookback_spin_limit(0)
    out = sr.mingru_forward(x, W, h0=h0, workspace=ws)
    assert _compare("fused", [out], [ref], sr.workspace_status(ws))
    sr.set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT)
    again = sr.mingru_forward(x, W, h0=h0, workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK and torch.equal(again, ref)


def test_minmax_give_up_is_flagged_and_recovers(zero_polls):
    """MinMax B=8, T=32768, D=192 (2736 tiles): a give-up shows in the status;
    with the default budget the result is the normal one again."""
    cfg = synth.CONFIGS[synth.MINMAX]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    say("forced time-outs: MinMax B=8 T=32768 D=192")
    r = synth.device_uniform(synth.MINMAX, "r", (B, T, D), -1.0, 1.0)
    s = synth.device_uniform(synth.MINMAX, "s", (B, T, D), -1.5, 0.5)
    x0 = synth.device_uniform(synth.MINMAX, "x0", (B, D), -1.0, 1.0)
    ws = _ws(sr.raw_library().minmax_scan_workspace_size(B, T, D))
    sr.set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT)
    ref = sr.minmax_scan(r, s, x0, workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    sr.set_lookback_spin_limit(0)
    out = sr.minmax_scan(r, s, x0, workspace=ws)
    status = sr.workspace_status(ws)
    say(f"MinMax: status {status}")
    assert status in (sr.SR_OK, sr.SR_ERR_LOOKBACK_TIMEOUT)
    if status == sr.SR_OK:
        assert torch.equal(out, ref)
    sr.set_lookback_spin_limit(sr.LOOKBACK_SPIN_LIMIT)
    again = sr.minmax_scan(r, s, x0, workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK and torch.equal(again, ref)
