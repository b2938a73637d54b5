"""GPU parity of the products on narrow tiles (17..512 rows, and up to 4096
rows when a 128 x 128 tiling would leave CUs idle and K <= 1024: the step
over a batch of streams, short forwards): tiles of 64 or 32 rows x 64
columns, the K range split over groups of waves inside the workgroup.  Shapes cover both
tile heights, ragged rows, columns, channels and K, K shorter than one
group's share, operands that allow no 16-byte loads, and full tiles."""

import numpy as np
import pytest
import torch

from oracle import decay, metrics, mingru
from tests.gpu_util import TOL_F32, dev, host64, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _weights(rng, D_in, D_h, D_out):
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / max(D_in, 1) ** 0.5).astype(np.float32)
    W_out = (rng.standard_normal((D_h, D_out)) / D_h ** 0.5).astype(np.float32)
    return W_in, W_out


@pytest.mark.parametrize("B,D_in,D_h,D_out", [
    (100, 40, 300, 130),      # 32-row tiles; K = 40: three K tiles over eight groups
    (300, 130, 333, 517),     # odd D_h and D_in: no 16-byte loads; ragged everything
    (480, 512, 1024, 1024),   # 64-row tiles, last row tile half full
    (512, 256, 2048, 2048),   # 64-row tiles, every tile full
    (64, 2048, 64, 48),       # a long K over few tiles
    (1000, 700, 333, 129),    # above 512 rows (K <= 1024): ragged rows, odd D_h
    (2048, 512, 512, 512),    # above 512 rows, every tile full
    # 64-row tiles split K over four waves, three stage buffers each: K giving
    # each wave one, two and three stages (the pipeline's short paths), and a
    # ragged K that leaves waves partial or empty shares
    (256, 64, 2048, 64),
    (256, 128, 2048, 64),
    (256, 192, 2048, 64),
    (256, 100, 2048, 64),
])
def test_narrow_step_matches_oracle(B, D_in, D_h, D_out):
    say(f"narrow step B={B} D_in={D_in} D_h={D_h} D_out={D_out}")
    rng = np.random.default_rng([1700, B, D_h])
    W_in, W_out = _weights(rng, D_in, D_h, D_out)
    h = dev(rng.standard_normal((B, D_h)).astype(np.float32))
    h_ref = host64(h)
    for t in range(2):
        x_t = rng.standard_normal((B, D_in)).astype(np.float32)
        y_t, h = sr.mingru_step(dev(x_t), dev(W_in), dev(W_out), h_prev=h)
        y_ref, h_ref = mingru.step(x_t, W_in, W_out, h_ref)
        e_h = metrics.max_abs_rel(host64(h), h_ref)
        e_y = metrics.y_rel_err(host64(y_t), y_ref, h_ref, W_out)
        say("step", t, "errors", e_h, e_y)
        assert e_h < TOL_F32 and e_y < TOL_F32
        h_ref = host64(h)


def test_narrow_step_decayed_and_repeatable():
    B, D_in, D_h = 200, 72, 96
    say("narrow decayed step")
    rng = np.random.default_rng(1701)
    W_in, _ = _weights(rng, D_in, D_h, D_h)
    lam = (10.0 ** rng.uniform(-3, 0, D_h)).astype(np.float32)
    dt = rng.exponential(1.0, B).astype(np.float32)
    dt[:3] = 1e6   # saturating gaps
    x_t = rng.standard_normal((B, D_in)).astype(np.float32)
    h0 = rng.standard_normal((B, D_h)).astype(np.float32)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(2):
        y, h = sr.mingru_step_decayed(dev(x_t), dev(W_in), decay_rate=dev(lam), delta_t=dev(dt),
                                      h_prev=dev(h0), saturated=sat)
        outs.append(h)
    assert torch.equal(outs[0], outs[1])
    _, h_ref = decay.step(x_t, W_in, lam, dt, None, h0)
    err = metrics.max_abs_rel(host64(outs[0]), h_ref)
    say("error", err)
    assert err < TOL_F32
    assert int(sat.item()) == int(decay.saturated(lam, dt))


@pytest.mark.parametrize("B,T,D_in,D_h,D_out", [
    (3, 100, 96, 96, 200),    # projections of 300 rows, ragged columns
    (1, 512, 64, 256, 64),    # 512 rows, full tiles
    (7, 19, 5, 70, 33),       # K = 5 and 70 (not multiples of 16)
    (3, 1000, 96, 300, 200),  # 3000 rows: narrow tiles replace an underfilled 128-row tiling
])
def test_narrow_forward_projections(B, T, D_in, D_h, D_out):
    say(f"narrow forward B={B} T={T} D_in={D_in} D_h={D_h} D_out={D_out}")
    rng = np.random.default_rng([1702, B, T])
    W_in, W_out = _weights(rng, D_in, D_h, D_out)
    x = rng.standard_normal((B, T, D_in)).astype(np.float32)
    y = sr.mingru_forward(dev(x), dev(W_in), W_out=dev(W_out))
    y2 = sr.mingru_forward(dev(x), dev(W_in), W_out=dev(W_out))
    assert torch.equal(y, y2)
    y_ref, h_ref, _ = mingru.layer(x, W_in, W_out)
    err = metrics.y_rel_err(host64(y), y_ref, h_ref, W_out)
    say("error", err)
    assert err < TOL_F32
