"""GPU parity of the fused projection + scan (taken by mingru_forward with W_in
when the problem has at least 512 tiles of 256 steps x 64 channels)."""

import numpy as np
import pytest
import torch

from oracle import decay, metrics, mingru
from tests.gpu_util import TOL_F32, dev, host64, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _fused_taken(B, T, D_in, D_h, D_out, with_out):
    """The fused path needs no [k|p] staging: adding W_in grows the workspace
    by less than that buffer alone."""
    size = sr.raw_library().mingru_forward_workspace_size
    grow = size(B, T, D_in, D_h, D_out, 1, int(with_out)) - size(B, T, 0, D_h, D_out, 0, int(with_out))
    return grow < B * T * 2 * D_h * 4


def _case(B, T, D_in, D_h, D_out, seed):
    rng = np.random.default_rng([1300, seed])
    x = rng.standard_normal((B, T, D_in)).astype(np.float32)
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / D_in ** 0.5).astype(np.float32)
    W_out = (rng.standard_normal((D_h, D_out)) / D_h ** 0.5).astype(np.float32)
    h0 = rng.standard_normal((B, D_h)).astype(np.float32)
    return x, W_in, W_out, h0


@pytest.mark.parametrize("B,T,D_in,D_h,D_out,with_out,with_h0", [
    (8, 1000, 64, 1024, 1024, True, True),     # ragged last tile along T
    (10, 777, 40, 1000, 1000, False, False),   # ragged along T and D, K not a multiple of 16
    (2, 4100, 16, 2048, 2048, False, True),    # a 4-step last tile
    (4, 2048, 96, 2048, 512, True, False),
    (1, 16384, 32, 512, 512, False, True),     # one batch row, 64 tiles along T
    (64, 5, 24, 512, 256, True, True),         # one partial tile per chain: 5 of 256 steps
])
def test_fused_forward_matches_oracle(B, T, D_in, D_h, D_out, with_out, with_h0):
    say(f"fused B={B} T={T} D_in={D_in} D_h={D_h} D_out={D_out} out={with_out} h0={with_h0}")
    assert _fused_taken(B, T, D_in, D_h, D_out, with_out)
    x, W_in, W_out, h0 = _case(B, T, D_in, D_h, D_out, seed=B + T + D_h)
    h0 = h0 if with_h0 else None
    Wo = W_out if with_out else None
    y, last = sr.mingru_forward(dev(x), dev(W_in), h0=None if h0 is None else dev(h0),
                                W_out=None if Wo is None else dev(Wo), return_last=True)
    k, p = mingru.layer_kp(x, W_in)
    h_ref = mingru.scan(k, p, h0)
    carry, inp = mingru.scan_terms(k, p, h0)
    if with_out:
        y_ref = mingru.project(h_ref, Wo)
        err = metrics.y_rel_err(host64(y), y_ref, h_ref, Wo)
    else:
        err = metrics.h_rel_err(host64(y), h_ref, carry, inp)
    last_err = metrics.h_rel_err(host64(last), h_ref[:, -1], carry[:, -1], inp[:, -1])
    say("errors", err, last_err)
    assert err < TOL_F32 and last_err < TOL_F32


def test_fused_forward_repeatable_and_carried():
    """Identical bits on repeated calls; two calls carrying h_T equal one call
    over the whole sequence (within rounding: the tiles fall differently)."""
    B, T, D_in, D_h = 8, 2048, 64, 1024
    x, W_in, _, h0 = _case(B, T, D_in, D_h, D_h, seed=7)
    xd, Wd, h0d = dev(x), dev(W_in), dev(h0)
    y1 = sr.mingru_forward(xd, Wd, h0=h0d)
    y2 = sr.mingru_forward(xd, Wd, h0=h0d)
    assert torch.equal(y1, y2)
    T1 = 1024
    assert _fused_taken(B, T1, D_in, D_h, D_h, False)
    a, la = sr.mingru_forward(xd[:, :T1].contiguous(), Wd, h0=h0d, return_last=True)
    b = sr.mingru_forward(xd[:, T1:].contiguous(), Wd, h0=la)
    assert metrics.max_abs_rel(host64(torch.cat([a, b], 1)), host64(y1)) < 1e-5


def test_fused_decayed_forward_matches_oracle():
    B, T, D_in, D_h = 8, 1000, 64, 1024
    say("fused decayed")
    assert _fused_taken(B, T, D_in, D_h, D_h, False)
    x, W_in, _, h0 = _case(B, T, D_in, D_h, D_h, seed=11)
    rng = np.random.default_rng(1301)
    lam = (10.0 ** rng.uniform(-3, 0, D_h)).astype(np.float32)
    dt = rng.exponential(1.0, (B, T)).astype(np.float32)
    dt[rng.random((B, T)) < 0.01] = 1e6
    for log1p in (False, True):
        sat = torch.zeros(1, dtype=torch.int32, device="cuda")
        h = sr.mingru_forward_decayed(dev(x), dev(W_in), decay_rate=dev(lam), delta_t=dev(dt),
                                      log1p_delta=log1p, saturated=sat, h0=dev(h0))
        k, p = mingru.layer_kp(x, W_in)
        ref = decay.scan(k, p, lam, dt, h0, log1p)
        carry, inp = decay.scan_terms(k, p, lam, dt, h0, log1p)
        err = metrics.h_rel_err(host64(h), ref, carry, inp)
        say("log1p", log1p, "error", err)
        assert err < TOL_F32
        assert int(sat.item()) == int(decay.saturated(lam, dt, log1p))


def test_fused_decayed_with_output_projection():
    """Decay, W_in and W_out together (the fused projection + scan, then the
    output GEMM) against the oracle layer."""
    B, T, D_in, D_h, D_out = 8, 1024, 48, 1024, 320
    say("fused decayed with W_out")
    assert _fused_taken(B, T, D_in, D_h, D_out, True)
    x, W_in, W_out, h0 = _case(B, T, D_in, D_h, D_out, seed=13)
    rng = np.random.default_rng(1302)
    lam = (10.0 ** rng.uniform(-2, 0, D_h)).astype(np.float32)
    dt = rng.exponential(0.5, (B, T)).astype(np.float32)
    y, last = sr.mingru_forward_decayed(dev(x), dev(W_in), decay_rate=dev(lam), delta_t=dev(dt),
                                        h0=dev(h0), W_out=dev(W_out), return_last=True)
    y_ref, h_ref, last_ref = decay.layer(x, W_in, lam, dt, W_out, h0)
    err = metrics.y_rel_err(host64(y), y_ref, h_ref, W_out)
    k, p = mingru.layer_kp(x, W_in)
    carry, inp = decay.scan_terms(k, p, lam, dt, h0)
    last_err = metrics.h_rel_err(host64(last), last_ref, carry[:, -1], inp[:, -1])
    say("errors", err, last_err)
    assert err < TOL_F32 and last_err < TOL_F32
