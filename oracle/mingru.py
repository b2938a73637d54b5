"""minGRU layer, run as its plain sequential definition in float64.

The method (the log-space minGRU layer of the "Mingru Pytorch" profile,
intro and "Requirements & limits"; the pages name the layer, its log-space
numerically stable form and its two modes, and print no equations, so the
minGRU recurrence they refer to is written out as stated):

    [k_t | p_t] = x_t W_in            k = first D_h columns, p = the next D_h
    z_t         = sigma(k_t)
    htilde_t    = g(p_t)
    h_t         = (1 - z_t) * h_{t-1} + z_t * htilde_t      t = 1..T
    y_t         = h_t W_out           (y_t = h_t when W_out is absent)

h_0 is the carried state; absent means zero (the profile's sequential guide
starts from a previous hidden state of None).  The parallel mode (guide
"Install and apply the minGRU layer") returns y for the whole sequence, the
sequential mode (guide "Process a sequence sequentially with carried hidden
state") takes one token and the previous hidden state and returns the output
and the next hidden state.

Pinned by: exact rational brute force of the linear recurrence, closed forms
(z = 1, z = 0, constant z, the convolution form), the log-space parallel form,
the convex-hull invariant and carried-state concatenation
(tests/test_oracle_mingru.py).  The projection is a library matmul pinned by
an explicit fsum dot product on a small case.
"""

from __future__ import annotations

import numpy as np

from . import scalar


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor (any dtype) -> float64 numpy
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def project(x, W):
    """x [..., K] @ W [K, N] in float64."""
    return np.matmul(_f64(x), _f64(W))


def split_kp(kp, D_h: int):
    """Column convention of [k | p] = x W_in: k first, then p."""
    return kp[..., :D_h], kp[..., D_h:2 * D_h]


def linear_recurrence(a, b, h0=None):
    """h_t = a_t * h_{t-1} + b_t over axis 1 of [B, T, D] arrays, float64."""
    a = _f64(a)
    b = _f64(b)
    B, T, D = a.shape
    h = np.zeros((B, D)) if h0 is None else _f64(h0).copy()
    out = np.empty((B, T, D))
    for t in range(T):
        h = a[:, t, :] * h + b[:, t, :]
        out[:, t, :] = h
    return out


def scan(k, p, h0=None):
    """The minGRU recurrence over t given the gate logits k and candidate
    pre-activations p ([B, T, D]); returns h [B, T, D] float64."""
    k = _f64(k)
    p = _f64(p)
    z = scalar.sigmoid(k)
    a = scalar.sigmoid(-k)  # = 1 - z (log(1 - z) = -softplus(k)), without cancelling
    htilde = scalar.g(p)
    B, T, D = k.shape
    h = np.zeros((B, D)) if h0 is None else _f64(h0).copy()
    out = np.empty((B, T, D))
    for t in range(T):
        h = a[:, t, :] * h + z[:, t, :] * htilde[:, t, :]
        out[:, t, :] = h
    return out


def scan_terms(k, p, h0=None):
    """The two terms of h_t = (prod_s (1 - z_s)) h_0 + (h_t with h_0 = 0).

    Returns (carry_mag, input_term): |prod (1 - z)| * |h_0| and the zero-state
    response, both float64 [B, T, D].  Their sum bounds the size of the
    quantities h_t is computed from, and conditions the relative error.
    """
    k = _f64(k)
    input_term = scan(k, p, None)
    if h0 is None:
        carry = np.zeros_like(input_term)
    else:
        decay = np.cumprod(scalar.sigmoid(-k), axis=1)  # prod (1 - z)
        carry = decay * np.abs(_f64(h0))[:, None, :]
    return carry, input_term


def layer(x, W_in, W_out=None, h0=None):
    """Parallel-mode layer: returns (y [B,T,D_out], h [B,T,D_h], h_last)."""
    W_in = _f64(W_in)
    D_h = W_in.shape[1] // 2
    kp = project(x, W_in)
    k, p = split_kp(kp, D_h)
    h = scan(k, p, h0)
    y = h if W_out is None else project(h, W_out)
    return y, h, h[:, -1, :].copy()


def layer_kp(x, W_in):
    """The projected gate logits and candidate pre-activations (k, p)."""
    W_in = _f64(W_in)
    D_h = W_in.shape[1] // 2
    return split_kp(project(x, W_in), D_h)


def step(x_t, W_in, W_out=None, h_prev=None):
    """Sequential mode, one token: x_t [B, D_in] -> (y_t [B, D_out], h_t [B, D_h])."""
    W_in = _f64(W_in)
    D_h = W_in.shape[1] // 2
    kp = project(x_t, W_in)
    k, p = split_kp(kp, D_h)
    z = scalar.sigmoid(k)
    htilde = scalar.g(p)
    h = np.zeros_like(z) if h_prev is None else _f64(h_prev)
    h_t = scalar.sigmoid(-k) * h + z * htilde  # sigma(-k) = 1 - z
    y_t = h_t if W_out is None else project(h_t, W_out)
    return y_t, h_t
