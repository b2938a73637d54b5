"""Oracle pins for the scans' gradients: fp64 autograd through independently
written forward loops, central finite differences, and closed forms; plus
planted mistakes that the pins must catch."""

import numpy as np
import pytest
import torch

from oracle import grad, scalar



def _mingru_inputs(seed, B=2, T=9, D=3, k_mean=0.0):
    rng = np.random.default_rng([1000, seed])
    k = rng.normal(k_mean, 1.5, (B, T, D))
    p = rng.normal(0.0, 1.5, (B, T, D))
    h0 = rng.normal(0.0, 1.0, (B, D))
    dh = rng.normal(0.0, 1.0, (B, T, D))
    dl = rng.normal(0.0, 1.0, (B, D))
    return k, p, h0, dh, dl


def _torch_mingru_loss(k, p, h0, dh, dl):
    z = torch.sigmoid(k)
    gp = torch.where(p >= 0, p + 0.5, torch.sigmoid(p))
    h = h0
    loss = 0.0
    for t in range(k.shape[1]):
        h = (1 - z[:, t]) * h + z[:, t] * gp[:, t]
        loss = loss + (dh[:, t] * h).sum()
    return loss + (dl * h).sum()


def autograd_mingru(k, p, h0, dh, dl):
    tk, tp, th = (torch.tensor(v, requires_grad=True) for v in (k, p, h0))
    _torch_mingru_loss(tk, tp, th, torch.tensor(dh), torch.tensor(dl)).backward()
    return tk.grad.numpy(), tp.grad.numpy(), th.grad.numpy()


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("seed,k_mean", [(0, 0.0), (1, -3.0), (2, 3.0)])
def test_mingru_backward_matches_autograd(seed, k_mean):
    k, p, h0, dh, dl = _mingru_inputs(seed, k_mean=k_mean)
    ours = grad.mingru_scan_backward(k, p, h0, dh, dl)
    ref = autograd_mingru(k, p, h0, dh, dl)
    for a, b in zip(ours, ref):
        assert _rel(a, b) < 1e-12


def test_mingru_backward_finite_differences():
    k, p, h0, dh, dl = _mingru_inputs(5, B=1, T=6, D=2)

    def loss(k_, p_, h0_):
        with torch.no_grad():
            return float(_torch_mingru_loss(torch.tensor(k_), torch.tensor(p_),
                                            torch.tensor(h0_), torch.tensor(dh), torch.tensor(dl)))
    dk, dp, dh0 = grad.mingru_scan_backward(k, p, h0, dh, dl)
    eps = 1e-6
    for arr, g in ((k, dk), (p, dp), (h0, dh0)):
        for idx in np.ndindex(arr.shape):
            if arr is p and abs(arr[idx]) < 1e-3:
                continue  # g has a kink in its derivative at p = 0
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = [plus if a is arr else a for a in (k, p, h0)]
            args_m = [minus if a is arr else a for a in (k, p, h0)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(g[idx])), (idx, fd, g[idx])


def test_mingru_backward_closed_forms():
    rng = np.random.default_rng(1010)
    B, T, D = 2, 50, 3
    p = rng.normal(0.0, 2.0, (B, T, D))
    h0 = rng.normal(0.0, 1.0, (B, D))
    dh = rng.normal(0.0, 1.0, (B, T, D))
    dl = rng.normal(0.0, 1.0, (B, D))
    # z = 0 (k = -40): every h_t is h_0, so dL/dh_0 collects every upstream gradient.
    dk, dp, dh0 = grad.mingru_scan_backward(np.full((B, T, D), -40.0), p, h0, dh, dl)
    assert np.allclose(dh0, dh.sum(axis=1) + dl, rtol=1e-13, atol=1e-13)
    assert np.max(np.abs(dk)) < 1e-15 and np.max(np.abs(dp)) < 1e-15
    # z = 1 exactly (k = +800: 1 - z = e^-800 / (1 + e^-800) is 0 in fp64; at
    # k = +40 it is 4e-18, not 0): h_t = g(p_t), nothing flows to h_0 or across steps.
    dk, dp, dh0 = grad.mingru_scan_backward(np.full((B, T, D), 800.0), p, h0, dh, dl)
    G = dh.copy()
    G[:, -1] += dl
    assert np.array_equal(dh0, np.zeros_like(dh0)) and np.array_equal(dk, np.zeros_like(dk))
    assert np.allclose(dp, G * grad.g_prime(p), rtol=1e-14, atol=0)


def test_g_prime_matches_derivative_of_g():
    x = np.array([-7.0, -1.0, -0.25, 0.25, 1.0, 5.0])
    eps = 1e-6
    fd = (scalar.g(x + eps) - scalar.g(x - eps)) / (2 * eps)
    assert np.max(np.abs(fd - grad.g_prime(x))) < 1e-9


def _minmax_inputs(seed, B=2, T=40, D=4):
    rng = np.random.default_rng([1020, seed])
    r = rng.uniform(-1, 1, (B, T, D))
    s = rng.uniform(-1, 1, (B, T, D)) - 0.5
    x0 = rng.uniform(-1, 1, (B, D))
    dx = rng.normal(0.0, 1.0, (B, T, D))
    dl = rng.normal(0.0, 1.0, (B, D))
    return r, s, x0, dx, dl


def _torch_minmax_loss(r, s, x0, dx, dl):
    x = x0
    loss = 0.0
    for t in range(r.shape[1]):
        x = torch.maximum(torch.minimum(r[:, t], x), s[:, t])
        loss = loss + (dx[:, t] * x).sum()
    return loss + (dl * x).sum()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_minmax_backward_matches_autograd(seed):
    r, s, x0, dx, dl = _minmax_inputs(seed)
    tr, ts, tx = (torch.tensor(v, requires_grad=True) for v in (r, s, x0))
    _torch_minmax_loss(tr, ts, tx, torch.tensor(dx), torch.tensor(dl)).backward()
    ours = grad.minmax_scan_backward(r, s, x0, dx, dl)
    for a, b in zip(ours, (tr.grad.numpy(), ts.grad.numpy(), tx.grad.numpy())):
        assert _rel(a, b) < 1e-14


def test_minmax_backward_finite_differences():
    r, s, x0, dx, dl = _minmax_inputs(7, B=1, T=8, D=2)

    def loss(r_, s_, x0_):
        with torch.no_grad():
            return float(_torch_minmax_loss(torch.tensor(r_), torch.tensor(s_), torch.tensor(x0_),
                                            torch.tensor(dx), torch.tensor(dl)))
    dr, ds, dx0 = grad.minmax_scan_backward(r, s, x0, dx, dl)
    eps = 1e-9  # piecewise linear: exact away from the kinks
    for arr, g in ((r, dr), (s, ds), (x0, dx0)):
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = [plus if a is arr else a for a in (r, s, x0)]
            args_m = [minus if a is arr else a for a in (r, s, x0)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-5, (idx, fd, g[idx])


def test_minmax_backward_closed_forms():
    rng = np.random.default_rng(1030)
    B, T, D = 2, 60, 3
    r = np.full((B, T, D), 2.0)
    s = np.full((B, T, D), -2.0)
    x0 = rng.uniform(-1, 1, (B, D))
    dx = rng.normal(0.0, 1.0, (B, T, D))
    dl = rng.normal(0.0, 1.0, (B, D))
    dr, ds, dx0 = grad.minmax_scan_backward(r, s, x0, dx, dl)  # nothing is ever selected
    assert not dr.any() and not ds.any()
    assert np.allclose(dx0, dx.sum(axis=1) + dl, rtol=1e-13, atol=1e-13)
    tstar = 23
    r[:, tstar] = -3.0
    s[:, tstar] = 0.5  # a forced reset to s_{t*}
    dr, ds, dx0 = grad.minmax_scan_backward(r, s, x0, dx, dl)
    assert not dr.any()
    assert np.allclose(ds[:, tstar], dx[:, tstar:].sum(axis=1) + dl, rtol=1e-13, atol=1e-13)
    assert np.allclose(dx0, dx[:, :tstar].sum(axis=1), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- mutations

def _mutant_mingru(drop_a=False, shift_h=False, wrong_gprime=False):
    def bwd(k, p, h0, dh, dh_last=None):
        z = scalar.sigmoid(k)
        a = 1 - z
        gp = scalar.g(p)
        B, T, D = k.shape
        h = h0.copy()
        hp = np.empty_like(k)
        for t in range(T):
            hp[:, t] = h
            h = a[:, t] * h + z[:, t] * gp[:, t]
        if shift_h:
            hp = np.concatenate([hp[:, 1:], h[:, None]], axis=1)
        gpr = np.ones_like(p) if wrong_gprime else grad.g_prime(p)
        dk = np.empty_like(k)
        dp = np.empty_like(k)
        G = dh_last.copy()
        for t in range(T - 1, -1, -1):
            G = dh[:, t] + G
            dk[:, t] = G * z[:, t] * a[:, t] * (gp[:, t] - hp[:, t])
            dp[:, t] = G * z[:, t] * gpr[:, t]
            G = G if drop_a else a[:, t] * G
        return dk, dp, G
    return bwd


@pytest.mark.parametrize("kw", [dict(drop_a=True), dict(shift_h=True), dict(wrong_gprime=True)])
def test_mingru_autograd_pin_catches_mistakes(kw):
    k, p, h0, dh, dl = _mingru_inputs(3)
    ours = _mutant_mingru(**kw)(k, p, h0, dh, dl)
    ref = autograd_mingru(k, p, h0, dh, dl)
    assert max(_rel(a, b) for a, b in zip(ours, ref)) > 1e-3


def test_minmax_autograd_pin_catches_wrong_selection():
    r, s, x0, dx, dl = _minmax_inputs(4)
    tr, ts, tx = (torch.tensor(v, requires_grad=True) for v in (r, s, x0))
    _torch_minmax_loss(tr, ts, tx, torch.tensor(dx), torch.tensor(dl)).backward()
    # swap the roles of r and s in the routing
    dr, ds, dx0 = grad.minmax_scan_backward(r, s, x0, dx, dl)
    assert _rel(ds, tr.grad.numpy()) > 1e-3 and _rel(dr, ts.grad.numpy()) > 1e-3


# ---------------------------------------------------------------- decayed

def _decay_inputs(seed, B=2, T=9, D=3):
    k, p, h0, dh, dl = _mingru_inputs(seed, B=B, T=T, D=D)
    rng = np.random.default_rng([1020, seed])
    lam = 10.0 ** rng.uniform(-2, 0, D)
    gap = rng.exponential(1.0, (B, T))
    return k, p, h0, dh, dl, lam, gap


def _torch_decayed_loss(k, p, h0, dh, dl, lam, gap):
    # Written independently of oracle/decay.py: gamma = exp(-min(lambda gap, 1e4)).
    z = torch.sigmoid(k)
    gp = torch.where(p >= 0, p + 0.5, torch.sigmoid(p))
    gam = torch.exp(-torch.clamp(gap[:, :, None] * lam[None, None, :], max=1e4))
    h = h0
    loss = 0.0
    for t in range(k.shape[1]):
        h = (1 - z[:, t]) * (gam[:, t] * h) + z[:, t] * gp[:, t]
        loss = loss + (dh[:, t] * h).sum()
    return loss + (dl * h).sum()


def autograd_decayed(k, p, h0, dh, dl, lam, gap):
    tk, tp, th = (torch.tensor(v, requires_grad=True) for v in (k, p, h0))
    _torch_decayed_loss(tk, tp, th, torch.tensor(dh), torch.tensor(dl), torch.tensor(lam),
                        torch.tensor(gap)).backward()
    return tk.grad.numpy(), tp.grad.numpy(), th.grad.numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decayed_backward_matches_autograd(seed):
    k, p, h0, dh, dl, lam, gap = _decay_inputs(seed)
    ours = grad.mingru_decayed_scan_backward(k, p, lam, gap, h0, dh, dl)
    ref = autograd_decayed(k, p, h0, dh, dl, lam, gap)
    for a, b in zip(ours, ref):
        assert _rel(a, b) < 1e-12


def test_decayed_backward_finite_differences():
    k, p, h0, dh, dl, lam, gap = _decay_inputs(5, B=1, T=6, D=2)

    def loss(k_, p_, h0_):
        with torch.no_grad():
            return float(_torch_decayed_loss(torch.tensor(k_), torch.tensor(p_), torch.tensor(h0_),
                                             torch.tensor(dh), torch.tensor(dl), torch.tensor(lam),
                                             torch.tensor(gap)))
    dk, dp, dh0 = grad.mingru_decayed_scan_backward(k, p, lam, gap, h0, dh, dl)
    eps = 1e-6
    for arr, g in ((k, dk), (p, dp), (h0, dh0)):
        for idx in np.ndindex(arr.shape):
            if arr is p and abs(arr[idx]) < 1e-3:
                continue
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = [plus if a is arr else a for a in (k, p, h0)]
            args_m = [minus if a is arr else a for a in (k, p, h0)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(g[idx])), (idx, fd, g[idx])


def test_decayed_backward_reduces_to_undecayed():
    # lambda = 0 or every gap 0: gamma = 1 exactly, the same arithmetic.
    k, p, h0, dh, dl, lam, gap = _decay_inputs(7)
    plain = grad.mingru_scan_backward(k, p, h0, dh, dl)
    for lam_, gap_ in ((np.zeros_like(lam), gap), (lam, np.zeros_like(gap))):
        dec = grad.mingru_decayed_scan_backward(k, p, lam_, gap_, h0, dh, dl)
        for a, b in zip(dec, plain):
            assert np.array_equal(a, b)


def test_decayed_backward_saturating_gap_cuts_the_gradient():
    # A gap of 1e6 at step t* (gamma = 0 there): nothing before t* feels the
    # gradients from t* on, and dh0 vanishes when t* is the first step.
    k, p, h0, dh, dl, lam, gap = _decay_inputs(8, T=12)
    ts = 5
    gap = gap.copy()
    gap[:, ts] = 1e6
    dk, dp, dh0 = grad.mingru_decayed_scan_backward(k, p, lam, gap, h0, dh, dl)
    dh2 = dh.copy()
    dh2[:, ts:] *= -3.0
    dk2, dp2, dh02 = grad.mingru_decayed_scan_backward(k, p, lam, gap, h0, dh2, 5.0 * dl)
    assert np.array_equal(dk[:, :ts], dk2[:, :ts]) and np.array_equal(dp[:, :ts], dp2[:, :ts])
    assert np.array_equal(dh0, dh02)
    gap[:, 0] = 1e6
    assert np.all(grad.mingru_decayed_scan_backward(k, p, lam, gap, h0, dh, dl)[2] == 0.0)


def test_decayed_backward_log1p_gaps():
    k, p, h0, dh, dl, lam, gap = _decay_inputs(9)
    u = gap
    a = grad.mingru_decayed_scan_backward(k, p, lam, np.expm1(u), h0, dh, dl, log1p_delta=True)
    b = grad.mingru_decayed_scan_backward(k, p, lam, u, h0, dh, dl)
    for x, y in zip(a, b):
        assert _rel(x, y) < 1e-13


def _mutant_decayed(k, p, lam, gap, h0, dh, dl, undecayed_dk=False, next_gamma=False,
                    no_gamma_in_g=False):
    """Planted mistakes: h_{t-1} undecayed in dk; gamma_{t+1} used where
    gamma_t belongs; G propagated without the decay."""
    from oracle import decay
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)
    gp = scalar.g(p)
    gam = decay.gamma(lam, gap)
    B, T, D = k.shape
    h = h0.copy()
    h_prev = np.empty((B, T, D))
    for t in range(T):
        h_prev[:, t] = h
        h = a[:, t] * (gam[:, t] * h) + z[:, t] * gp[:, t]
    dk = np.empty((B, T, D))
    G = dl.copy()
    for t in range(T - 1, -1, -1):
        G = dh[:, t] + G
        gt = gam[:, min(t + 1, T - 1)] if next_gamma else gam[:, t]
        dk[:, t] = G * z[:, t] * a[:, t] * (gp[:, t] - (1.0 if undecayed_dk else gt) * h_prev[:, t])
        G = a[:, t] * (1.0 if no_gamma_in_g else gam[:, t]) * G
    return dk, G


@pytest.mark.parametrize("kw", [dict(undecayed_dk=True), dict(next_gamma=True),
                                dict(no_gamma_in_g=True)])
def test_decayed_autograd_pin_catches_mistakes(kw):
    k, p, h0, dh, dl, lam, gap = _decay_inputs(3)
    dk_ref, _, dh0_ref = autograd_decayed(k, p, h0, dh, dl, lam, gap)
    dk, dh0 = _mutant_decayed(k, p, lam, gap, h0, dh, dl, **kw)
    assert _rel(dk, dk_ref) > 1e-6 or _rel(dh0, dh0_ref) > 1e-6
    # and the unmutated arithmetic passes the same check
    dk0, dh00 = _mutant_decayed(k, p, lam, gap, h0, dh, dl)
    assert _rel(dk0, dk_ref) < 1e-12 and _rel(dh00, dh0_ref) < 1e-12
