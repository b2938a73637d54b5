"""GPU parity of the scans' backward pass against the fp64 oracle."""

import numpy as np
import pytest
import torch

import synth
from oracle import grad, scalar
from tests.gpu_util import dev, host64, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")

TOL = 1e-4


def _abs_G(k, dh, dh_last):
    """|G|-bound: the reverse recurrence run on |dh| (every term non-negative)."""
    a = scalar.sigmoid(-np.asarray(k, np.float64))  # 1 - sigma(k)
    B, T, D = k.shape
    G = np.zeros((B, D)) if dh_last is None else np.abs(dh_last)
    out = np.empty((B, T, D))
    for t in range(T - 1, -1, -1):
        G = np.abs(dh[:, t]) + G
        out[:, t] = G
        G = a[:, t] * G
    return out


def _mingru_errors(k, p, h0, dh, dl, dk, dp, dh0):
    """Conditioned errors: |d - d_ref| / (|G| z (1-z) (|g| + |h_prev|)) for dk and
    |d - d_ref| / (|G| z |g'|) for dp, with |G| from _abs_G."""
    k = np.asarray(k, np.float64)
    p = np.asarray(p, np.float64)
    rdk, rdp, rdh0 = grad.mingru_scan_backward(k, p, h0, dh, dl)
    Gabs = _abs_G(k, dh, dl)
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)  # 1 - z
    g = scalar.g(p)
    B, T, D = k.shape
    h = np.zeros((B, D)) if h0 is None else np.asarray(h0, np.float64).copy()
    hp = np.empty_like(k)
    for t in range(T):
        hp[:, t] = h
        h = a[:, t] * h + z[:, t] * g[:, t]
    den_k = Gabs * z * a * (np.abs(g) + np.abs(hp)) + 1e-30
    den_p = Gabs * z * grad.g_prime(p) + 1e-30
    e_k = float(np.max(np.abs(host64(dk) - rdk) / den_k))
    e_p = float(np.max(np.abs(host64(dp) - rdp) / den_p))
    e_0 = 0.0
    if dh0 is not None:
        e_0 = float(np.max(np.abs(host64(dh0) - rdh0) / (a[:, 0] * Gabs[:, 0] + 1e-30)))
    return e_k, e_p, e_0


@pytest.mark.parametrize("B,T,D,with_h0,with_last", [
    (2, 64, 16, False, False),
    (3, 1000, 200, True, True),
    (2, 4096, 512, True, False),
    (1, 1, 8, True, True),
    (2, 3, 3, False, True),
    (1, 777, 130, True, True),
])
def test_mingru_backward_f32(B, T, D, with_h0, with_last):
    say(f"mingru bwd f32 B={B} T={T} D={D}")
    rng = np.random.default_rng([1100, B, T, D])
    k = rng.normal(-1.0, 1.5, (B, T, D)).astype(np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32) if with_h0 else None
    dh = rng.standard_normal((B, T, D)).astype(np.float32)
    dl = rng.standard_normal((B, D)).astype(np.float32) if with_last else None
    kd, pd = dev(k), dev(p)
    h0d = None if h0 is None else dev(h0)
    h = sr.mingru_forward(k=kd, p=pd, h0=h0d)
    dk, dp, dh0 = sr.mingru_scan_backward(kd, pd, h, dev(dh), h0=h0d,
                                          dh_last=None if dl is None else dev(dl))
    errs = _mingru_errors(k, p, h0, dh, dl, dk, dp, dh0)
    say("errors", errs)
    assert max(errs) < TOL, errs


def test_mingru_backward_bf16_long_memory_reduced():
    B, T, D = 2, 4096, 1024
    say("mingru bwd bf16")
    cfg = synth.CONFIGS[synth.SCAN]
    k32 = synth.normal_bt(synth.SCAN, "k", B, T, D, cfg["k_mean"], cfg["k_std"])
    p32 = synth.normal_bt(synth.SCAN, "p", B, T, D, cfg["p_mean"], cfg["p_std"])
    kb, pb = synth.bf16_round(k32).cuda(), synth.bf16_round(p32).cuda()
    h0 = synth.normal_vec(synth.SCAN, "h0", B, D)
    rng = np.random.default_rng(1101)
    dh = rng.standard_normal((B, T, D)).astype(np.float32)
    dl = rng.standard_normal((B, D)).astype(np.float32)
    h = sr.mingru_forward(k=kb, p=pb, h0=dev(h0))
    dk, dp, dh0 = sr.mingru_scan_backward(kb, pb, h, dev(dh), h0=dev(h0), dh_last=dev(dl))
    errs = _mingru_errors(kb.double().cpu().numpy(), pb.double().cpu().numpy(), h0, dh, dl,
                          dk, dp, dh0)
    say("errors", errs)
    assert max(errs) < 1e-4, errs


def test_mingru_backward_repeatable():
    B, T, D = 2, 5000, 256
    rng = np.random.default_rng(1102)
    kd = dev(rng.normal(-2.0, 1.0, (B, T, D)).astype(np.float32))
    pd = dev(rng.standard_normal((B, T, D)).astype(np.float32))
    dh = dev(rng.standard_normal((B, T, D)).astype(np.float32))
    h = sr.mingru_forward(k=kd, p=pd)
    ref = sr.mingru_scan_backward(kd, pd, h, dh)
    for _ in range(2):
        again = sr.mingru_scan_backward(kd, pd, h, dh)
        assert torch.equal(again[0], ref[0]) and torch.equal(again[1], ref[1])


def _minmax_case(B, T, D, seed):
    rng = np.random.default_rng([1110, seed])
    r = rng.uniform(-1, 1, (B, T, D)).astype(np.float32)
    s = (rng.uniform(-1, 1, (B, T, D)) - 0.5).astype(np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    for a in (r, s, x0):
        a[a == 0] = 0.0
    dx = rng.standard_normal((B, T, D)).astype(np.float32)
    dl = rng.standard_normal((B, D)).astype(np.float32)
    return r, s, x0, dx, dl


@pytest.mark.parametrize("B,T,D", [(2, 64, 16), (3, 1000, 200), (1, 1, 5), (2, 5000, 192),
                                   (4, 333, 7)])
def test_minmax_backward(B, T, D):
    say(f"minmax bwd B={B} T={T} D={D}")
    r, s, x0, dx, dl = _minmax_case(B, T, D, seed=B + T + D)
    rd, sd, x0d = dev(r), dev(s), dev(x0)
    x_out = sr.minmax_scan(rd, sd, x0d)
    dr, ds, dx0 = sr.minmax_scan_backward(rd, sd, x0d, x_out, dev(dx), dx_last=dev(dl))
    rdr, rds, rdx0 = grad.minmax_scan_backward(r, s, x0, dx, dl)
    # The routing (which operand each step selects) is decided exactly.
    assert np.array_equal(host64(dr) != 0, rdr != 0)
    assert np.array_equal(host64(ds) != 0, rds != 0)
    # The routed values are sums of upstream gradients: fp32 sums.
    scale = np.abs(dx).sum(axis=1).max() + np.abs(dl).max()
    for got, ref in ((dr, rdr), (ds, rds), (dx0, rdx0)):
        assert float(np.max(np.abs(host64(got) - ref))) < 1e-5 * scale


def test_minmax_backward_hold_and_reset():
    B, T, D = 2, 20000, 192
    rng = np.random.default_rng(1120)
    r = np.full((B, T, D), 2.0, np.float32)
    s = np.full((B, T, D), -2.0, np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    tstar = 12345
    r[:, tstar] = -3.0
    s[:, tstar] = 0.5
    dx = np.ones((B, T, D), np.float32)  # sums of ones are exact in fp32
    rd, sd, x0d = dev(r), dev(s), dev(x0)
    x_out = sr.minmax_scan(rd, sd, x0d)
    dr, ds, dx0 = sr.minmax_scan_backward(rd, sd, x0d, x_out, dev(dx))
    assert torch.count_nonzero(dr) == 0
    assert torch.all(dx0 == float(tstar))
    assert torch.all(ds[:, tstar] == float(T - tstar))
    assert torch.count_nonzero(ds) == B * D


def test_full_size_b8_t65536_d1024_backward_every_element():
    """The backward at the bench workload's full size: dk, dp and dh0 of every
    channel and step against the fp64 oracle's gradients (worker processes)."""
    from tests import fullsize
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    say("full size B=8 T=65536 D=1024 backward, every element")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    g = torch.Generator(device="cuda")
    g.manual_seed(1130)
    dh = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    h = sr.mingru_forward(k=kb, p=pb, h0=h0)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    dk, dp, dh0 = sr.mingru_scan_backward(kb, pb, h, dh, h0=h0, workspace=ws)
    assert sr.workspace_status(ws) == 0
    assert bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dp).all())
    H = fullsize.host32
    arrays = dict(k=H(kb), p=H(pb), h0=H(h0), dh=H(dh), dk=H(dk), dp=H(dp), dh0=H(dh0))
    del kb, pb, h, dh, dk, dp
    torch.cuda.empty_cache()
    say("oracle gradients on every channel")
    res = fullsize.all_channels(fullsize.backward_slice_errors, arrays, B, D)
    errs = tuple(max(r[i] for r in res) for i in range(3))
    say("full size backward errors (every element)", errs)
    assert max(errs) < 1e-4, errs


def test_mingru_backward_extreme_values():
    """Gate logits up to |k| = 87 (both sigmoids stay normal fp32 numbers),
    candidates up to 1e30, against the fp64 oracle with the conditioned
    errors (their floors keep outputs far below the fp32 range out of the
    relative measure); the workspace status stays clear."""
    rng = np.random.default_rng(1140)
    B, T, D = 2, 2000, 130
    k = rng.choice([-87.0, -80.0, -30.0, -3.0, 0.0, 3.0, 30.0, 80.0, 87.0], (B, T, D)).astype(np.float32)
    p = rng.choice([-1e4, -100.0, -20.0, -1.0, 0.0, 1.0, 20.0, 1e6, 1e30], (B, T, D)).astype(np.float32)
    h0 = rng.choice([-1e6, -1.0, 0.0, 1.0, 1e6], (B, D)).astype(np.float32)
    dh = rng.standard_normal((B, T, D)).astype(np.float32)
    dl = rng.standard_normal((B, D)).astype(np.float32)
    say("mingru bwd extremes")
    kd, pd, h0d = dev(k), dev(p), dev(h0)
    h = sr.mingru_forward(k=kd, p=pd, h0=h0d)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    dk, dp, dh0 = sr.mingru_scan_backward(kd, pd, h, dev(dh), h0=h0d, dh_last=dev(dl), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_OK
    assert bool(torch.isfinite(dk).all() and torch.isfinite(dp).all() and torch.isfinite(dh0).all())
    errs = _mingru_errors(k, p, h0, dh, dl, dk, dp, dh0)
    say("errors", errs)
    assert max(errs) < TOL, errs


def test_mingru_backward_gate_logits_past_the_fp32_range():
    """|k| up to 1e4 in the backward: the flushed factors drop terms below
    1e-35 with moderate candidates and states, the gradients still meet the
    bar, and the backward reports the range in its workspace status."""
    rng = np.random.default_rng(1141)
    B, T, D = 2, 2000, 130
    k = rng.choice([-1e4, -100.0, -88.0, -4.0, 0.0, 4.0, 88.0, 100.0, 1e4], (B, T, D)).astype(np.float32)
    p = rng.choice([-20.0, -1.0, 0.0, 1.0, 20.0, 1e3], (B, T, D)).astype(np.float32)
    h0 = rng.choice([-1e3, -1.0, 0.0, 1.0, 1e3], (B, D)).astype(np.float32)
    dh = rng.standard_normal((B, T, D)).astype(np.float32)
    dl = rng.standard_normal((B, D)).astype(np.float32)
    say("mingru bwd past the range")
    kd, pd, h0d = dev(k), dev(p), dev(h0)
    h = sr.mingru_forward(k=kd, p=pd, h0=h0d)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    dk, dp, dh0 = sr.mingru_scan_backward(kd, pd, h, dev(dh), h0=h0d, dh_last=dev(dl), workspace=ws)
    assert sr.workspace_status(ws) == sr.SR_ERR_GATE_RANGE
    assert bool(torch.isfinite(dk).all() and torch.isfinite(dp).all() and torch.isfinite(dh0).all())
    errs = _mingru_errors(k, p, h0, dh, dl, dk, dp, dh0)
    say("errors", errs)
    assert max(errs) < TOL, errs


def test_mingru_backward_kp_halves_of_one_buffer():
    """k and p as the two halves of one [B,T,2D] buffer (row stride 2D, as the
    input projection writes them): the same gradients as from separate
    contiguous tensors, bit for bit, and the oracle's."""
    B, T, D = 2, 3000, 192
    say("mingru bwd kp halves")
    rng = np.random.default_rng(4100)
    kp = rng.standard_normal((B, T, 2 * D)).astype(np.float32)
    kp[..., :D] -= 2.0
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    dh = rng.standard_normal((B, T, D)).astype(np.float32)
    kpd = dev(kp)
    k_view, p_view = kpd[..., :D], kpd[..., D:]
    h = sr.mingru_forward(k=k_view, p=p_view, h0=dev(h0))
    got = sr.mingru_scan_backward(k_view, p_view, h, dev(dh), h0=dev(h0))
    sep = sr.mingru_scan_backward(k_view.contiguous(), p_view.contiguous(), h, dev(dh), h0=dev(h0))
    for a, b in zip(got, sep):
        assert torch.equal(a, b)
    k, p = kp[..., :D], kp[..., D:]
    errs = _mingru_errors(k, p, h0, dh, None, *got)
    say("errors", errs)
    assert max(errs) < TOL


def test_backward_two_chains_across_eight_thousand_tiles():
    """B=1, T=2^18, D=256: two chains of 4096 tiles each, with ~256 tiles of
    each chain in flight at once, so nearly every tile walks back through
    predecessors word by word (the backward's serial look-back) -- against
    the oracle on sampled channels over the whole sequence."""
    B, T, D = 1, 1 << 18, 256
    say(f"backward, two chains: B={B} T={T} D={D}")
    g = torch.Generator(device="cuda")
    g.manual_seed(1140)
    k = (torch.empty((B, T, D), device="cuda").normal_(-3.0, 1.0, generator=g)).to(torch.bfloat16)
    p = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g).to(torch.bfloat16)
    h0 = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    dh = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    dl = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    h = sr.mingru_forward(k=k, p=p, h0=h0)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    dk, dp, dh0 = sr.mingru_scan_backward(k, p, h, dh, h0=h0, dh_last=dl, workspace=ws)
    assert sr.workspace_status(ws) == 0
    ds = torch.as_tensor([0, 127, 128, 255], device="cuda")  # both tiles' edges
    sl = lambda t: t[0][:, ds].double().cpu().numpy()[None]
    errs = _mingru_errors(sl(k), sl(p), h0[0][ds].double().cpu().numpy()[None], sl(dh),
                          dl[0][ds].double().cpu().numpy()[None],
                          dk[0][:, ds][None], dp[0][:, ds][None], dh0[0][ds][None])
    say("errors", errs)
    assert max(errs) < TOL, errs
