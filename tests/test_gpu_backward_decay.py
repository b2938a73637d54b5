"""GPU parity of the time-decayed scan's backward pass against the fp64 oracle
(oracle/grad.py, mingru_decayed_scan_backward)."""

import numpy as np
import pytest
import torch

import synth
from oracle import decay, grad, scalar
from tests.gpu_util import dev, host64, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")

TOL = 1e-4


def _decay_errors(k, p, h0, dh, dl, lam, gap, log1p, dk, dp, dh0):
    """Conditioned errors, as for the undecayed backward with the coefficient
    a_t gamma_t: |G| is the reverse recurrence on |dh|, and the dk scale is
    |G| z a (|g| + gamma |h_prev|)."""
    k = np.asarray(k, np.float64)
    p = np.asarray(p, np.float64)
    rdk, rdp, rdh0 = grad.mingru_decayed_scan_backward(k, p, lam, gap, h0, dh, dl, log1p)
    gam = decay.gamma(lam, gap, log1p)
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)
    g = scalar.g(p)
    B, T, D = k.shape
    h = np.zeros((B, D)) if h0 is None else np.asarray(h0, np.float64).copy()
    hp = np.empty_like(k)
    for t in range(T):
        hp[:, t] = h
        h = a[:, t] * (gam[:, t] * h) + z[:, t] * g[:, t]
    Gabs = np.empty_like(k)
    G = np.zeros((B, D)) if dl is None else np.abs(np.asarray(dl, np.float64))
    for t in range(T - 1, -1, -1):
        G = np.abs(dh[:, t]) + G
        Gabs[:, t] = G
        G = a[:, t] * gam[:, t] * G
    den_k = Gabs * z * a * (np.abs(g) + gam * np.abs(hp)) + 1e-30
    den_p = Gabs * z * grad.g_prime(p) + 1e-30
    e_k = float(np.max(np.abs(host64(dk) - rdk) / den_k))
    e_p = float(np.max(np.abs(host64(dp) - rdp) / den_p))
    e_0 = 0.0
    if dh0 is not None:
        e_0 = float(np.max(np.abs(host64(dh0) - rdh0) / (a[:, 0] * gam[:, 0] * Gabs[:, 0] + 1e-30)))
    return e_k, e_p, e_0


def _case(B, T, D, seed, huge_every=0):
    rng = np.random.default_rng([1300, B, T, D, seed])
    k = rng.normal(-1.0, 1.5, (B, T, D)).astype(np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    dh = rng.standard_normal((B, T, D)).astype(np.float32)
    dl = rng.standard_normal((B, D)).astype(np.float32)
    lam = (10.0 ** rng.uniform(-3, 0, D)).astype(np.float32)
    gap = rng.exponential(1.0, (B, T)).astype(np.float32)
    if huge_every:
        gap[:, ::huge_every] = 1e6  # saturating gaps: gamma = 0, the gradient is cut
    return k, p, h0, dh, dl, lam, gap


@pytest.mark.parametrize("B,T,D,with_h0,log1p,huge_every", [
    (2, 64, 16, True, False, 0),
    (3, 1000, 200, True, False, 97),    # two channels per lane, ragged T and D
    (1, 777, 333, False, True, 0),      # odd D: one channel per lane; log1p gaps
    (2, 4096, 512, True, False, 1000),  # many tiles, cut gradients
    (1, 1, 8, True, False, 1),          # one step with a saturating gap
])
def test_decayed_backward_f32(B, T, D, with_h0, log1p, huge_every):
    say(f"decayed bwd f32 B={B} T={T} D={D} log1p={log1p} huge_every={huge_every}")
    k, p, h0, dh, dl, lam, gap = _case(B, T, D, 1, huge_every)
    h0 = h0 if with_h0 else None
    kd, pd = dev(k), dev(p)
    h0d = None if h0 is None else dev(h0)
    h = sr.mingru_forward_decayed(k=kd, p=pd, h0=h0d, decay_rate=dev(lam), delta_t=dev(gap),
                                  log1p_delta=log1p)
    dk, dp, dh0 = sr.mingru_scan_backward_decayed(kd, pd, h, dev(dh), h0=h0d, dh_last=dev(dl),
                                                  decay_rate=dev(lam), delta_t=dev(gap),
                                                  log1p_delta=log1p)
    errs = _decay_errors(k, p, h0, dh, dl, lam, gap, log1p, dk, dp, dh0)
    say("errors", errs)
    assert max(errs) < TOL, errs


def test_zero_rate_equals_undecayed_backward_bitwise():
    B, T, D = 2, 3000, 256
    say("decayed bwd, zero rate = undecayed")
    k, p, h0, dh, dl, lam, gap = _case(B, T, D, 2)
    kd, pd, h0d, dhd, dld = dev(k), dev(p), dev(h0), dev(dh), dev(dl)
    h = sr.mingru_forward(k=kd, p=pd, h0=h0d)
    plain = sr.mingru_scan_backward(kd, pd, h, dhd, h0=h0d, dh_last=dld)
    dec = sr.mingru_scan_backward_decayed(kd, pd, h, dhd, h0=h0d, dh_last=dld,
                                          decay_rate=torch.zeros(D, device="cuda"),
                                          delta_t=dev(gap))
    for a, b in zip(dec, plain):
        assert torch.equal(a, b)


def test_full_size_b8_t65536_d1024_decayed_backward_every_element():
    """The decayed scan's backward at the headline scan's shape (bf16 k/p):
    dk, dp and dh0 of every channel and step against the fp64 oracle's
    gradients (worker processes)."""
    from tests import fullsize
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    say("decayed bwd full size B=8 T=65536 D=1024, every element")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    lam = torch.as_tensor(synth.decay_rates(synth.SCAN, D), device="cuda")
    gap = torch.as_tensor(synth.gaps(synth.SCAN, B, T), device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1301)
    dh = torch.empty((B, T, D), device="cuda").normal_(0.0, 1.0, generator=g)
    dl = torch.empty((B, D), device="cuda").normal_(0.0, 1.0, generator=g)
    h = sr.mingru_forward_decayed(k=kb, p=pb, h0=h0, decay_rate=lam, delta_t=gap)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    dk, dp, dh0 = sr.mingru_scan_backward_decayed(kb, pb, h, dh, h0=h0, dh_last=dl, workspace=ws,
                                                  decay_rate=lam, delta_t=gap)
    assert sr.workspace_status(ws) == 0
    assert bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dp).all())
    H = fullsize.host32
    arrays = dict(k=H(kb), p=H(pb), h0=H(h0), dh=H(dh), dh_last=H(dl), dk=H(dk), dp=H(dp),
                  dh0=H(dh0), lam=H(lam), dt=H(gap), log1p=np.zeros(1, np.int32))
    del kb, pb, h, dh, dk, dp
    torch.cuda.empty_cache()
    say("oracle gradients on every channel")
    res = fullsize.all_channels(fullsize.backward_slice_errors, arrays, B, D)
    errs = tuple(max(r[i] for r in res) for i in range(3))
    say("decayed backward errors (every element)", errs)
    assert max(errs) < TOL, errs


@pytest.mark.parametrize("decayed", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_autograd_scan_uses_the_backward_kernels(decayed, dtype):
    """sr.mingru_scan under torch autograd: the gradients of k, p and h0 are
    the backward kernels' results, bit for bit."""
    B, T, D = 2, 1500, 256
    say(f"autograd scan decayed={decayed} dtype={dtype}")
    k, p, h0, dh, _, lam, gap = _case(B, T, D, 3, 300)
    kd = dev(k).to(dtype).requires_grad_()
    pd = dev(p).to(dtype).requires_grad_()
    h0d = dev(h0).requires_grad_()
    dhd = dev(dh)
    kw = dict(decay_rate=dev(lam), delta_t=dev(gap)) if decayed else {}
    h = sr.mingru_scan(kd, pd, h0d, **kw)
    (h * dhd).sum().backward()
    fn = sr.mingru_scan_backward_decayed if decayed else sr.mingru_scan_backward
    with torch.no_grad():
        ref = fn(kd.detach(), pd.detach(), h.detach(), dhd, h0=h0d.detach(), **kw)
    assert torch.equal(kd.grad, ref[0].to(dtype)) and torch.equal(pd.grad, ref[1].to(dtype))
    assert torch.equal(h0d.grad, ref[2])
