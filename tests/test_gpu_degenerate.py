"""GPU parity of the degenerate sizes the layer admits: no input features
(D_in = 0, so k = p = 0 and the recurrence is h_t = h_{t-1} / 2 + 1 / 4),
on every projection path (fused with the scan, narrow tiles, large tiles, the
small-batch FMA path, the step), and a zero-width state with an output
projection (y = 0)."""

import numpy as np
import pytest
import torch

from oracle import mingru, metrics
from tests.gpu_util import TOL_F32, dev, host64, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


@pytest.mark.parametrize("B,T,D_h,with_out", [
    (8, 1024, 1024, False),   # projection fused with the scan (512 tiles)
    (2, 100, 64, True),       # 200 rows: narrow tiles
    (4, 1000, 256, True),     # 4000 rows: large tiles
])
def test_forward_without_input_features(B, T, D_h, with_out):
    say(f"D_in=0 forward B={B} T={T} D_h={D_h} out={with_out}")
    rng = np.random.default_rng([1800, B, T])
    x = np.zeros((B, T, 0), np.float32)
    W_in = np.zeros((0, 2 * D_h), np.float32)
    W_out = (rng.standard_normal((D_h, 48)) / D_h ** 0.5).astype(np.float32) if with_out else None
    h0 = rng.standard_normal((B, D_h)).astype(np.float32)
    y, last = sr.mingru_forward(dev(x), dev(W_in), h0=dev(h0),
                                W_out=None if W_out is None else dev(W_out), return_last=True)
    y_ref, h_ref, last_ref = mingru.layer(x, W_in, W_out, h0)
    if with_out:
        err = metrics.y_rel_err(host64(y), y_ref, h_ref, W_out)
    else:
        err = metrics.max_abs_rel(host64(y), h_ref)
    say("error", err)
    assert err < TOL_F32
    assert metrics.max_abs_rel(host64(last), last_ref) < TOL_F32


@pytest.mark.parametrize("B,D_h", [(4, 96), (256, 2048), (1024, 512)])
def test_step_without_input_features(B, D_h):
    say(f"D_in=0 step B={B} D_h={D_h}")
    rng = np.random.default_rng([1801, B])
    h0 = rng.standard_normal((B, D_h)).astype(np.float32)
    x_t = np.zeros((B, 0), np.float32)
    W_in = np.zeros((0, 2 * D_h), np.float32)
    _, h = sr.mingru_step(dev(x_t), dev(W_in), h_prev=dev(h0))
    _, h_ref = mingru.step(x_t, W_in, None, h0)
    assert metrics.max_abs_rel(host64(h), h_ref) < TOL_F32
    assert np.allclose(h_ref, 0.5 * h0.astype(np.float64) + 0.25)


def test_zero_width_state_with_output_projection():
    B, T, D_in, D_out = 2, 9, 5, 7
    say("D_h=0 with W_out")
    x = dev(np.ones((B, T, D_in), np.float32))
    y = sr.mingru_forward(x, dev(np.zeros((D_in, 0), np.float32)),
                          W_out=dev(np.zeros((0, D_out), np.float32)))
    assert y.shape == (B, T, D_out) and torch.count_nonzero(y) == 0
