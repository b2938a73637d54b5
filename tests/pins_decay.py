"""Pins for the time-decayed recurrence: checks against things other than the
oracle itself.  Each pin takes the scan under test,
``scan(k, p, decay_rate, delta_t, h0=None, log1p_delta=False)``, so the same
pin runs against the oracle and against copies of it with a planted mistake.

* page_example_err -- "Your first delta model", Step 5: the same token fed six
                      times; a zero gap is no decay; after a saturating gap
                      the state is back to its value after the first event
                      and the next events repeat; decay only ever shrinks the
                      state of this all-positive example.
* no_decay_err     -- a zero rate or a zero gap is the plain minGRU scan.
* closed_const_err -- constant inputs per channel: a geometric series, with
                      rates varying over channels and gaps over batch rows.
* rational_err     -- exact rational brute force with gamma = 2^-n.
* log1p_err        -- delta_t = expm1(u) with log1p_delta equals delta_t = u.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

PAGE_GAPS = [0.0, 1.0, 1.0, 20000.0, 1.0, 1.0]


def page_case(D=8, seed=0):
    """k, p of one recurring token (B=1, T=6), and a rate per channel large
    enough that the 20000 gap saturates (lambda * 20000 > 1e4)."""
    rng = np.random.default_rng([900, seed])
    k1 = rng.normal(0.0, 1.0, D)
    p1 = rng.normal(0.0, 1.0, D)
    k = np.broadcast_to(k1, (1, 6, D)).copy()
    p = np.broadcast_to(p1, (1, 6, D)).copy()
    lam = rng.uniform(0.6, 2.0, D)
    return k, p, lam


def page_example_err(scan, no_decay_scan):
    """0.0 when every property of the page's worked example holds, else > 0."""
    k, p, lam = page_case()
    gapped = np.array([PAGE_GAPS])
    control = np.zeros_like(gapped)
    hg = scan(k, p, lam, gapped)[0]
    hc = scan(k, p, lam, control)[0]
    plain = no_decay_scan(k, p)[0]
    err = 0.0
    # Control: gamma = exp(0) = 1, i.e. exactly the undecayed recurrence.
    err += float(np.max(np.abs(hc - plain)))
    # The first event has a zero gap in both schedules.
    err += float(np.max(np.abs(hg[0] - hc[0])))
    # After the huge gap the state restarts: events 3, 4, 5 repeat 0, 1, 2.
    err += float(np.max(np.abs(hg[3:6] - hg[0:3])))
    ng, nc = np.linalg.norm(hg, axis=1), np.linalg.norm(hc, axis=1)
    # Control accumulates monotonically; the gapped norms at events 1, 2 are
    # below control's (the decay shrinks a positive state).
    err += float(np.sum(np.maximum(nc[:-1] - nc[1:], 0.0)))
    err += float(np.sum(np.maximum(ng[1:3] - nc[1:3] + 1e-12, 0.0)))
    return err


def no_decay_err(scan, no_decay_scan, seed=1):
    rng = np.random.default_rng([901, seed])
    B, T, D = 2, 40, 5
    k = rng.normal(-0.5, 1.5, (B, T, D))
    p = rng.normal(0.0, 1.0, (B, T, D))
    h0 = rng.normal(0.0, 1.0, (B, D))
    ref = no_decay_scan(k, p, h0)
    zero_gap = scan(k, p, rng.uniform(0.1, 3.0, D), np.zeros((B, T)), h0)
    zero_rate = scan(k, p, np.zeros(D), rng.uniform(0.0, 50.0, (B, T)), h0)
    return float(max(np.max(np.abs(zero_gap - ref)), np.max(np.abs(zero_rate - ref))))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _g(x):
    return np.where(x >= 0, x + 0.5, _sigmoid(x))


def closed_const_err(scan, seed=2):
    """k, p constant per channel, gaps constant per batch row, B == D so a
    rate/gap swap still broadcasts and has to be caught by value.
    h_t = c^t h0 + q (1 - c^t) / (1 - c), c = (1 - z) e^{-lambda gap}, q = z g."""
    rng = np.random.default_rng([902, seed])
    B = D = 3
    T = 25
    kd = rng.normal(0.0, 1.0, D)
    pd = rng.normal(0.0, 1.0, D)
    lam = np.array([0.05, 0.4, 1.3])
    gap = np.array([0.2, 1.0, 3.0])
    h0 = rng.normal(0.0, 1.0, (B, D))
    k = np.broadcast_to(kd, (B, T, D)).copy()
    p = np.broadcast_to(pd, (B, T, D)).copy()
    dt = np.broadcast_to(gap[:, None], (B, T)).copy()
    h = scan(k, p, lam, dt, h0)
    z = _sigmoid(kd)
    c = (1.0 - z)[None, :] * np.exp(-gap[:, None] * lam[None, :])   # [B, D]
    q = (z * _g(pd))[None, :]
    err = 0.0
    for t in range(1, T + 1):
        carry, inp = c ** t * h0, q * (1.0 - c ** t) / (1.0 - c)
        den = np.abs(carry) + np.abs(inp)
        err = max(err, float(np.max(np.abs(h[:, t - 1] - (carry + inp)) / den)))
    return err


def rational_err(scan, seed=3):
    """z in {1/4, 1/2, 3/4}, g(p) = p + 1/2 with dyadic p >= 0, and
    lambda_d = m_d ln 2 with integer gaps n, so gamma = 2^{-m_d n} and the
    recurrence runs exactly in rationals."""
    rng = np.random.default_rng([903, seed])
    B, T, D = 2, 30, 4
    zs = [Fraction(1, 4), Fraction(1, 2), Fraction(3, 4)]
    zi = rng.integers(0, 3, (B, T, D))
    pn = rng.integers(0, 9, (B, T, D))          # p = pn / 8
    m = np.array([1, 2, 1, 3])
    n = rng.integers(0, 4, (B, T))
    h0n = rng.integers(0, 9, (B, D))            # h0 = h0n / 4 >= 0: well conditioned
    k = np.log(np.array([[[float(zs[i] / (1 - zs[i])) for i in row] for row in blk]
                         for blk in zi]))
    p = pn / 8.0
    lam = m * np.log(2.0)
    h = scan(k, p, lam, n.astype(np.float64), h0n / 4.0)
    err = 0.0
    for b in range(B):
        for d in range(D):
            x = Fraction(int(h0n[b, d]), 4)
            for t in range(T):
                z = zs[zi[b, t, d]]
                gamma = Fraction(1, 2 ** (int(m[d]) * int(n[b, t])))
                x = (1 - z) * gamma * x + z * (Fraction(int(pn[b, t, d]), 8) + Fraction(1, 2))
                err = max(err, abs(h[b, t, d] - float(x)) / max(abs(float(x)), 1e-300))
    return err


def log1p_err(scan, seed=4):
    rng = np.random.default_rng([904, seed])
    B, T, D = 2, 30, 4
    k = rng.normal(0.0, 1.0, (B, T, D))
    p = rng.normal(0.0, 1.0, (B, T, D))
    lam = rng.uniform(0.1, 2.0, D)
    u = rng.uniform(0.0, 3.0, (B, T))
    a = scan(k, p, lam, np.expm1(u), None, log1p_delta=True)
    b = scan(k, p, lam, u, None)
    return float(np.max(np.abs(a - b) / (np.abs(b) + 1e-300)))
