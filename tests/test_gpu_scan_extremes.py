"""GPU scan tests at the edges: tile-geometry invariance (the tiling is a
performance-only choice, like the delta tutorial's `chunk_size`), one very
long look-back chain, and outputs larger than 4 GiB (64-bit offsets)."""

import numpy as np
import pytest
import torch

from oracle import metrics, minmax, mingru
from tests.gpu_util import TOL_F32, dev, host64, say, scan_err

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def test_mingru_result_does_not_depend_on_tile_geometry():
    """Two channels per lane (contiguous rows) against one channel per lane
    (rows with an odd stride force it): both match the oracle, and agree
    with each other to rounding."""
    B, T, D = 2, 3000, 256
    say("geometry invariance minGRU")
    rng = np.random.default_rng(900)
    k = rng.normal(-1.0, 1.5, (B, T, D)).astype(np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    y2 = sr.mingru_forward(k=dev(k), p=dev(p), h0=dev(h0))
    buf = torch.zeros((B, T, 2 * D + 1), device="cuda")
    buf[..., :D] = dev(k)
    buf[..., D + 1:] = dev(p)
    kk, pp = buf[..., :D], buf[..., D + 1:]
    assert kk.stride(1) == 2 * D + 1  # odd row stride: one channel per lane
    y1 = sr.mingru_forward(k=kk, p=pp, h0=dev(h0))
    assert scan_err(host64(y2), k, p, h0) < TOL_F32
    assert scan_err(host64(y1), k, p, h0) < TOL_F32
    assert float((y1 - y2).abs().max()) < 1e-5


def test_minmax_result_does_not_depend_on_tile_geometry():
    """D = 192 runs with one channel per lane, D = 194 with two; the first
    192 channels must be bit-identical, and equal to the oracle."""
    B, T = 3, 5000
    say("geometry invariance MinMax")
    rng = np.random.default_rng(901)
    r = rng.uniform(-1, 1, (B, T, 194)).astype(np.float32)
    s = (rng.uniform(-1, 1, (B, T, 194)) - 0.5).astype(np.float32)
    x0 = rng.uniform(-1, 1, (B, 194)).astype(np.float32)
    for a in (r, s, x0):
        a[a == 0] = 0.0
    wide = sr.minmax_scan(dev(r), dev(s), dev(x0))
    narrow = sr.minmax_scan(dev(r[..., :192]), dev(s[..., :192]), dev(x0[:, :192]))
    assert torch.equal(wide[..., :192], narrow)
    ref, _ = minmax.scan(r[..., :192], s[..., :192], x0[:, :192])
    assert metrics.bits_equal(narrow.cpu().numpy(), ref)


def test_one_long_lookback_chain():
    """B = 1 and D = 128 give a single chain of ~7300 tiles along
    T = 2^20; four channels are checked over the whole sequence."""
    B, T, D = 1, 1 << 20, 128
    say("long chain T=2^20")
    g = torch.Generator(device="cuda")
    g.manual_seed(902)
    k = torch.empty((B, T, D), device="cuda").normal_(-3.0, 1.0, generator=g)
    p = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    h0 = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    y, last = sr.mingru_forward(k=k, p=p, h0=h0, return_last=True, workspace=ws)
    assert sr.workspace_status(ws) == 0
    ch = [0, 37, 64, 127]
    kk = k[0, :, ch].double().cpu().numpy()[None]
    pp = p[0, :, ch].double().cpu().numpy()[None]
    hh = h0[0, ch].double().cpu().numpy()[None]
    err = scan_err(y[0, :, ch].double().cpu().numpy()[None], kk, pp, hh)
    say("long chain err", err)
    assert err < TOL_F32


def test_output_beyond_4_gib():
    """B = 16, T = 65536, D = 1024: h is 4 GiB, so element offsets pass 2^32
    bytes; sampled channels near the end are checked against the oracle."""
    B, T, D = 16, 65536, 1024
    say("h beyond 4 GiB")
    g = torch.Generator(device="cuda")
    g.manual_seed(903)
    k = torch.empty((B, T, D), device="cuda").normal_(-4.0, 1.0, generator=g).to(torch.bfloat16)
    p = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g).to(torch.bfloat16)
    h0 = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    y, last = sr.mingru_forward(k=k, p=p, h0=h0, return_last=True)
    bs = torch.tensor([15, 15, 14, 0], device="cuda")
    ds = torch.tensor([1023, 512, 7, 0], device="cuda")
    kk = k[bs, :, ds].double().cpu().numpy()[None].transpose(0, 2, 1)
    pp = p[bs, :, ds].double().cpu().numpy()[None].transpose(0, 2, 1)
    hh = h0[bs, ds].double().cpu().numpy()[None]
    got = y[bs, :, ds].double().cpu().numpy()[None].transpose(0, 2, 1)
    err = scan_err(got, kk, pp, hh)
    say("4 GiB err", err)
    assert err < 1e-5
    assert torch.equal(last, y[:, -1])
    del k, p, y
    torch.cuda.empty_cache()


def test_extreme_gate_and_candidate_values():
    """Gate logits deep into both saturations, candidates from -1e4 to 1e30
    and carried states up to 1e20, against the fp64 oracle: no NaN, no
    overflow, the conditioned error within the fp32 bar.  For |k| <= 87 both
    sigma(k) and sigma(-k) are normal fp32 numbers, so no term is dropped and
    the workspace status stays clear."""
    rng = np.random.default_rng(1600)
    B, T, D = 2, 3000, 130
    k_vals = np.array([-87.0, -80.0, -30.0, -3.0, 0.0, 3.0, 30.0, 80.0, 87.0])
    p_vals = np.array([-1e4, -100.0, -20.0, -1.0, 0.0, 1.0, 20.0, 1e6, 1e30])
    k = rng.choice(k_vals, (B, T, D)).astype(np.float32)
    p = rng.choice(p_vals, (B, T, D)).astype(np.float32)
    h0 = rng.choice([-1e20, -1.0, 0.0, 1.0, 1e20], (B, D)).astype(np.float32)
    say("extreme values")
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    h = sr.mingru_forward(k=dev(k), p=dev(p), h0=dev(h0), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    assert bool(torch.isfinite(h).all())
    # Outputs far below the fp32 normal range (e.g. sigma(-100) = 4e-44) are
    # flushed to zero: the error is measured against at least 1e-30.
    h_ref = mingru.scan(k, p, h0)
    carry, inp = mingru.scan_terms(k, p, h0)
    err = metrics.h_rel_err(host64(h), h_ref, carry, inp, floor=1e-30)
    say("error", err)
    assert err < TOL_F32


def test_gate_logits_past_the_fp32_range():
    """|k| up to 1e4: beyond ~87.3 the smaller of sigma(k), sigma(-k) flushes
    to zero in fp32 and the term it multiplies is dropped, which the scan
    reports (SR_ERR_GATE_RANGE) while still writing finite results.  With
    candidates and states of moderate size the dropped terms are below
    1e-35, so the results still meet the bar against the fp64 oracle."""
    rng = np.random.default_rng(1601)
    B, T, D = 2, 3000, 130
    k_vals = np.array([-1e4, -300.0, -100.0, -88.0, -87.0, -4.0, 0.0, 4.0, 87.0, 88.0, 100.0,
                       300.0, 1e4])
    k = rng.choice(k_vals, (B, T, D)).astype(np.float32)
    p = rng.choice([-20.0, -1.0, 0.0, 1.0, 20.0, 1e3], (B, T, D)).astype(np.float32)
    h0 = rng.choice([-1e3, -1.0, 0.0, 1.0, 1e3], (B, D)).astype(np.float32)
    say("gate logits past the fp32 range")
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    h = sr.mingru_forward(k=dev(k), p=dev(p), h0=dev(h0), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_ERR_GATE_RANGE
    assert bool(torch.isfinite(h).all())
    h_ref = mingru.scan(k, p, h0)
    carry, inp = mingru.scan_terms(k, p, h0)
    err = metrics.h_rel_err(host64(h), h_ref, carry, inp, floor=1e-30)
    say("error", err)
    assert err < TOL_F32
    # The same inputs with every |k| clipped to 87 are inside the range.
    kc = np.clip(k, -87.0, 87.0)
    sr.mingru_forward(k=dev(kc), p=dev(p), h0=dev(h0), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK


def test_dropped_term_is_reported():
    """Where the dropped term is the whole signal -- every gate at k = -100
    (sigma(k) = 3.7e-44, below the fp32 normal range) with candidates of 1e30
    from a zero state, so that h_t = t * 3.7e-14 in fp64 -- the fp32 result
    loses it (zero, or what is left of a subnormal factor), and the status
    says why.  One channel in range alongside is unaffected."""
    B, T, D = 1, 500, 64
    k = np.full((B, T, D), -100.0, np.float32)
    p = np.full((B, T, D), 1e30, np.float32)
    k[..., 0] = -2.0
    p[..., 0] = 1.0
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    h = sr.mingru_forward(k=dev(k), p=dev(p), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_ERR_GATE_RANGE
    lost = host64(h[..., 1:])
    full = mingru.scan(k[..., 1:2], p[..., 1:2])
    assert np.all(np.isfinite(lost)) and np.all(lost >= 0) and np.all(lost <= full * (1 + 1e-6))
    ref = mingru.scan(k[..., :1], p[..., :1])
    assert np.max(np.abs(host64(h[..., :1]) - ref) / ref) < TOL_F32


@pytest.mark.parametrize("T", [512, 65536])  # the GEMM + scan path, and the fused one
def test_gate_range_reported_through_the_layer(T):
    """A layer forward whose projection produces gate logits past the range
    (a weight column of 1e3 on inputs of size ~1) reports it too, on the
    fused path (2 x 65536 x 64: 512 tiles) and the unfused one."""
    B, D_in, D = 2, 16, 64
    rng = np.random.default_rng([1602, T])
    x = rng.standard_normal((B, T, D_in)).astype(np.float32)
    W = (rng.standard_normal((D_in, 2 * D)) / 4).astype(np.float32)
    nb = sr.raw_library().mingru_forward_workspace_size(B, T, D_in, D, D, 1, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sr.mingru_forward(dev(x), dev(W), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    W[:, 5] = 1e3
    y = sr.mingru_forward(dev(x), dev(W), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_ERR_GATE_RANGE
    assert bool(torch.isfinite(y).all())
