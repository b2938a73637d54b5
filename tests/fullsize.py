"""Full-size parity helpers: the oracle on every channel of a full-size
workload, in worker processes (oracle.parallel), and the per-slice error
tasks the workers run.  Each task reads its slice of the inputs and of the
GPU result from shared memory and returns the slice's conditioned errors."""

from __future__ import annotations

import numpy as np

from oracle import decay, grad, metrics, mingru, parallel, scalar

WIDTH = 64  # channels per slice of work


def _sl(arrays, name, sl, batched=True):
    b, d0, d1 = sl
    a = arrays[name]
    if a.ndim == 3:
        return np.asarray(a[b:b + 1, :, d0:d1], np.float64)
    if batched:  # [B, D]
        return np.asarray(a[b:b + 1, d0:d1], np.float64)
    return np.asarray(a[d0:d1], np.float64)  # [D]


def _gaps_row(arrays, sl):
    b, _, _ = sl
    return np.asarray(arrays["dt"][b:b + 1], np.float64)


# ---------------------------------------------------------------- forward

def decayed_slice_error(arrays, sl):
    k, p, h0 = _sl(arrays, "k", sl), _sl(arrays, "p", sl), _sl(arrays, "h0", sl)
    lam, dt = _sl(arrays, "lam", sl, batched=False), _gaps_row(arrays, sl)
    log1p = bool(arrays["log1p"][0])
    ref = decay.scan(k, p, lam, dt, h0, log1p)
    carry, inp = decay.scan_terms(k, p, lam, dt, h0, log1p)
    return metrics.h_rel_err(_sl(arrays, "got", sl), ref, carry, inp)


# --------------------------------------------------------------- backward

def _abs_G(coef, dh, dh_last):
    """|G|-bound: the reverse recurrence run on |dh| with the (non-negative)
    coefficients, every term non-negative."""
    B, T, D = dh.shape
    G = np.zeros((B, D)) if dh_last is None else np.abs(dh_last)
    out = np.empty((B, T, D))
    for t in range(T - 1, -1, -1):
        G = np.abs(dh[:, t]) + G
        out[:, t] = G
        G = coef[:, t] * G
    return out


def mingru_backward_errors(k, p, h0, dh, dh_last, dk, dp, dh0, lam=None, dt=None, log1p=False):
    """Conditioned errors of (dk, dp, dh0) against the oracle's gradients:
    |d - d_ref| / (|G| z (1 - z) (|g| + gamma |h_prev|)) for dk, / (|G| z g')
    for dp, / (coef_1 |G_1|) for dh0, with |G| the reverse recurrence on
    |dh| (its floors keep values far below the fp32 range out of the
    relative measure).  Time decay when lam (and dt) are given."""
    k = np.asarray(k, np.float64)
    p = np.asarray(p, np.float64)
    dh = np.asarray(dh, np.float64)
    if lam is None:
        rdk, rdp, rdh0 = grad.mingru_scan_backward(k, p, h0, dh, dh_last)
        gam = np.ones_like(k)
    else:
        rdk, rdp, rdh0 = grad.mingru_decayed_scan_backward(k, p, lam, dt, h0, dh, dh_last, log1p)
        gam = np.broadcast_to(decay.gamma(lam, dt, log1p), k.shape)
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)  # 1 - z
    coef = a * gam
    Gabs = _abs_G(coef, dh, dh_last)
    g = scalar.g(p)
    B, T, D = k.shape
    h = np.zeros((B, D)) if h0 is None else np.asarray(h0, np.float64).copy()
    hp = np.empty_like(k)
    for t in range(T):
        hp[:, t] = gam[:, t] * h
        h = a[:, t] * hp[:, t] + z[:, t] * g[:, t]
    den_k = Gabs * z * a * (np.abs(g) + np.abs(hp)) + 1e-30
    den_p = Gabs * z * grad.g_prime(p) + 1e-30
    e_k = float(np.max(np.abs(np.asarray(dk, np.float64) - rdk) / den_k))
    e_p = float(np.max(np.abs(np.asarray(dp, np.float64) - rdp) / den_p))
    e_0 = 0.0
    if dh0 is not None:
        e_0 = float(np.max(np.abs(np.asarray(dh0, np.float64) - rdh0) / (coef[:, 0] * Gabs[:, 0] + 1e-30)))
    return e_k, e_p, e_0


def backward_slice_errors(arrays, sl):
    lam = dt = None
    log1p = False
    if "lam" in arrays:
        lam, dt = _sl(arrays, "lam", sl, batched=False), _gaps_row(arrays, sl)
        log1p = bool(arrays["log1p"][0])
    dl = _sl(arrays, "dh_last", sl) if "dh_last" in arrays else None
    return mingru_backward_errors(_sl(arrays, "k", sl), _sl(arrays, "p", sl), _sl(arrays, "h0", sl),
                                  _sl(arrays, "dh", sl), dl, _sl(arrays, "dk", sl),
                                  _sl(arrays, "dp", sl), _sl(arrays, "dh0", sl), lam, dt, log1p)


def all_channels(task, arrays, B, D, workers=None):
    """task on every (batch row, 64-channel) slice, in worker processes."""
    return parallel.map_slices(task, arrays, parallel.channel_slices(B, D, WIDTH), workers)


def host32(t):
    """A GPU tensor as a float32 host array (bf16 values are exact in fp32)."""
    return t.detach().float().cpu().numpy()
