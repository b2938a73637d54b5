"""Gradients of the two scans, by the chain rule run backward in time (fp64).

The layers are trained (the minGRU profile's "Requirements & limits" names an
enwik8 training entry point; the minmaxrnc page, "Key properties", states that
gradients through the MinMax state path can neither vanish nor explode), so
the scans' backward pass is the next step of the hot path.  For an upstream
gradient dh_t = dL/dh_t on every output (and dh_last on the returned h_T):

minGRU, with a_t = 1 - z_t, z_t = sigma(k_t), b_t = z_t g(p_t):
    G_t      = dh_t + a_{t+1} G_{t+1}          (G_T = dh_T + dh_last)
    dL/dk_t  = G_t z_t (1 - z_t) (g(p_t) - h_{t-1})
    dL/dp_t  = G_t z_t g'(p_t),   g'(p) = 1 (p >= 0), sigma(p)(1 - sigma(p)) (p < 0)
    dL/dh_0  = a_1 G_1

MinMax, x_{t+1} = max(min(r_t, x_t), s_t): the output selects one operand.
Reading for ties (measure zero for continuous inputs): s_t is selected only if
strictly greater than min(r_t, x_t), and r_t only if strictly smaller than x_t;
otherwise the carried state passes through.
    Gamma_{t+1} = dx_{t+1} + [step t+1 passes its state] Gamma_{t+2}
    dL/dr_t = Gamma_{t+1} [r_t selected],  dL/ds_t = Gamma_{t+1} [s_t selected]
    dL/dx_0 = [step 0 passes its state] Gamma_1

Time-decayed minGRU (the decay contract of the "Your first delta model"
tutorial, Step 5 "Adding time decay": the carried state is scaled by
gamma_t = exp(-min(lambda_d gap_t, 1e4)) at the token boundary, as in
oracle/decay.py): the step's coefficient becomes c_t = a_t gamma_t, so
    G_t      = dh_t + c_{t+1} G_{t+1}
    dL/dk_t  = G_t z_t (1 - z_t) (g(p_t) - gamma_t h_{t-1})
    dL/dp_t  = G_t z_t g'(p_t)
    dL/dh_0  = c_1 G_1
with the rates and gaps held fixed (no gradient for them).

Pinned by: fp64 torch.autograd through independently written forward loops,
central finite differences, and closed forms (tests/test_oracle_grad.py).
"""

from __future__ import annotations

import numpy as np

from . import scalar
from .mingru import _f64


def g_prime(p):
    p = _f64(p)
    s = scalar.sigmoid(p)
    return np.where(p >= 0, 1.0, s * (1.0 - s))


def mingru_scan_backward(k, p, h0, dh, dh_last=None):
    """Returns (dk, dp, dh0) for L = sum_t <dh_t, h_t> + <dh_last, h_T>."""
    k = _f64(k)
    p = _f64(p)
    dh = _f64(dh)
    B, T, D = k.shape
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)  # = 1 - z, without cancelling
    gp = scalar.g(p)
    # forward states h_{t-1} entering each step
    h = np.zeros((B, D)) if h0 is None else _f64(h0).copy()
    h_prev = np.empty((B, T, D))
    for t in range(T):
        h_prev[:, t] = h
        h = a[:, t] * h + z[:, t] * gp[:, t]
    dk = np.empty((B, T, D))
    dp = np.empty((B, T, D))
    G = np.zeros((B, D)) if dh_last is None else _f64(dh_last).copy()
    for t in range(T - 1, -1, -1):
        G = dh[:, t] + G
        dk[:, t] = G * z[:, t] * a[:, t] * (gp[:, t] - h_prev[:, t])
        dp[:, t] = G * z[:, t] * g_prime(p[:, t])
        G = a[:, t] * G  # the part of dL/dh_{t-1} that flows through step t
    return dk, dp, G


def mingru_decayed_scan_backward(k, p, decay_rate, delta_t, h0, dh, dh_last=None,
                                 log1p_delta=False):
    """Returns (dk, dp, dh0) of the time-decayed scan (oracle/decay.py) for
    L = sum_t <dh_t, h_t> + <dh_last, h_T>; decay_rate [D], delta_t [B, T]."""
    from . import decay
    k = _f64(k)
    p = _f64(p)
    dh = _f64(dh)
    B, T, D = k.shape
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)
    gp = scalar.g(p)
    gam = decay.gamma(decay_rate, delta_t, log1p_delta)  # [B, T, D]
    h = np.zeros((B, D)) if h0 is None else _f64(h0).copy()
    h_prev = np.empty((B, T, D))
    for t in range(T):
        h_prev[:, t] = h
        h = a[:, t] * (gam[:, t] * h) + z[:, t] * gp[:, t]
    dk = np.empty((B, T, D))
    dp = np.empty((B, T, D))
    G = np.zeros((B, D)) if dh_last is None else _f64(dh_last).copy()
    for t in range(T - 1, -1, -1):
        G = dh[:, t] + G
        dk[:, t] = G * z[:, t] * a[:, t] * (gp[:, t] - gam[:, t] * h_prev[:, t])
        dp[:, t] = G * z[:, t] * g_prime(p[:, t])
        G = a[:, t] * gam[:, t] * G
    return dk, dp, G


def minmax_selection(r, s, x_prev):
    """0 = the carried state passes, 1 = r_t selected, 2 = s_t selected."""
    m = np.minimum(r, x_prev)
    return np.where(s > m, 2, np.where(r < x_prev, 1, 0))


def minmax_scan_backward(r, s, x0, dx, dx_last=None):
    """Returns (dr, ds, dx0) for L = sum_t <dx_t, x_out[t]> + <dx_last, x_T>."""
    r = np.asarray(r)
    s = np.asarray(s)
    B, T, D = r.shape
    x = np.array(x0, dtype=r.dtype, copy=True)
    sel = np.empty((B, T, D), dtype=np.int8)
    for t in range(T):
        sel[:, t] = minmax_selection(r[:, t], s[:, t], x)
        x = np.maximum(np.minimum(r[:, t], x), s[:, t])
    dx = _f64(dx)
    dr = np.zeros((B, T, D))
    ds = np.zeros((B, T, D))
    G = np.zeros((B, D)) if dx_last is None else _f64(dx_last).copy()
    for t in range(T - 1, -1, -1):
        G = G + dx[:, t]
        dr[:, t] = np.where(sel[:, t] == 1, G, 0.0)
        ds[:, t] = np.where(sel[:, t] == 2, G, 0.0)
        G = np.where(sel[:, t] == 0, G, 0.0)
    return dr, ds, G
