"""Time-decayed minGRU recurrence over a vector state, run sequentially in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Your first delta model" (the minGRU tutorials, chris-santiago.github.io),
Step 5 "Adding time decay".  What the page fixes:

* every mixer takes the same decay contract (decay="fixed"/"learnable" plus a
  per-event gap delta_t, the gap *preceding* each event);
* the carried state is multiplied by gamma_t once per token, at the token
  boundary, *before* that token's own write, which itself is not decayed;
* a zero gap gives gamma = exp(0) = 1, i.e. no decay;
* when lambda * delta_t exceeds about 1e4 the float32 computation saturates:
  the token's memory is wiped completely (handled by a clamp) and a warning
  is raised; with log1p_delta the gaps are compressed and the warning does
  not fire on the page's example (a 20000 gap).

Readings (the page shows a matrix-state mixer; this is the same contract on
the minGRU's vector state, and the page leaves these details open):

    gap_t   = log1p(delta_t) if log1p_delta else delta_t          (per b, t)
    e_t,d   = min(lambda_d * gap_t, 1e4)                          (the clamp)
    gamma   = exp(-e)
    h_t     = (1 - z_t) * (gamma_t * h_{t-1}) + z_t * g(p_t)
    saturated: some lambda_d * gap_t > 1e4, decided in float32 (the precision
               the page's warning speaks of and the GPU kernel works in).

lambda_d >= 0 is a per-channel rate (the page's "fixed" or "learnable" rate;
how a trainable rate is parameterised is the caller's business), delta_t >= 0
is finite.  exp(-1e4) is 0 in float64 and in float32, so the clamp changes no
value: a saturated token starts from a zero state, as if the sequence began
there.

Pinned by (tests/test_oracle_decay.py): the page's worked example (a huge gap
returns the state to exactly its value after the first event, and the next
events repeat; one saturation with raw gaps, none with log1p_delta; a zero gap
is no decay); the decay-free special case (lambda = 0 or delta_t = 0 gives the
plain minGRU recurrence); closed forms with constant inputs per channel
(geometric series, with rates varying over channels and gaps over rows, so a
transposed operand fails); exact rational brute force with gamma = 2^-n; the
log1p reparameterisation (delta_t = expm1(u) with log1p_delta equals delta_t =
u without); carried-state concatenation.
"""

from __future__ import annotations

import numpy as np

from . import mingru, scalar

SATURATION = 1.0e4


def _f64(a):
    return mingru._f64(a)


def gaps(delta_t, log1p_delta=False):
    """The gap each token decays by: delta_t, or log1p(delta_t) when compressed."""
    d = _f64(delta_t)
    return np.log1p(d) if log1p_delta else d


def exponent(decay_rate, delta_t, log1p_delta=False):
    """e[b, t, d] = min(lambda_d * gap[b, t], 1e4), float64."""
    lam = _f64(decay_rate)
    gap = gaps(delta_t, log1p_delta)
    return np.minimum(gap[:, :, None] * lam[None, None, :], SATURATION)


def gamma(decay_rate, delta_t, log1p_delta=False):
    """The per-token decay factor exp(-e), float64 [B, T, D]."""
    return np.exp(-exponent(decay_rate, delta_t, log1p_delta))


def saturated(decay_rate, delta_t, log1p_delta=False) -> bool:
    """Whether some token's lambda * gap exceeds the clamp, decided in float32."""
    lam = np.asarray(_f64(decay_rate), np.float32)
    gap = np.asarray(gaps(delta_t, log1p_delta), np.float32)
    prod = gap.reshape(-1)[:, None] * lam[None, :]  # float32 products, rounded once
    return bool(np.any(prod > np.float32(SATURATION)))


def scan(k, p, decay_rate, delta_t, h0=None, log1p_delta=False):
    """h [B, T, D] of the decayed recurrence, one token at a time."""
    k = _f64(k)
    p = _f64(p)
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)  # = 1 - z, without cancelling
    htilde = scalar.g(p)
    gam = gamma(decay_rate, delta_t, log1p_delta)
    B, T, D = k.shape
    h = np.zeros((B, D)) if h0 is None else _f64(h0).copy()
    out = np.empty((B, T, D))
    for t in range(T):
        h = gam[:, t, :] * h                               # the token boundary
        h = a[:, t, :] * h + z[:, t, :] * htilde[:, t, :]  # the token's write
        out[:, t, :] = h
    return out


def scan_terms(k, p, decay_rate, delta_t, h0=None, log1p_delta=False):
    """(|prod (1 - z) gamma| |h_0|, response to a zero h_0): the sizes of the two
    non-negative terms h is the sum of, for the conditioned error measure."""
    k = _f64(k)
    input_term = scan(k, p, decay_rate, delta_t, None, log1p_delta)
    if h0 is None:
        return np.zeros_like(input_term), input_term
    coef = np.cumprod(scalar.sigmoid(-k) * gamma(decay_rate, delta_t, log1p_delta), axis=1)
    return coef * np.abs(_f64(h0))[:, None, :], input_term


def layer(x, W_in, decay_rate, delta_t, W_out=None, h0=None, log1p_delta=False):
    """Parallel-mode layer with decay: (y, h, h_last)."""
    k, p = mingru.layer_kp(x, W_in)
    h = scan(k, p, decay_rate, delta_t, h0, log1p_delta)
    y = h if W_out is None else mingru.project(h, W_out)
    return y, h, h[:, -1, :].copy()


def step(x_t, W_in, decay_rate, delta_t, W_out=None, h_prev=None, log1p_delta=False):
    """One token: x_t [B, D_in], delta_t [B] -> (y_t, h_t)."""
    k, p = mingru.layer_kp(x_t, W_in)
    z = scalar.sigmoid(k)
    gam = gamma(decay_rate, _f64(delta_t)[:, None], log1p_delta)[:, 0, :]
    h = np.zeros_like(z) if h_prev is None else _f64(h_prev)
    h_t = scalar.sigmoid(-_f64(k)) * (gam * h) + z * scalar.g(p)
    y_t = h_t if W_out is None else mingru.project(h_t, W_out)
    return y_t, h_t
