"""The minGRU recurrence in its log-space parallel form, float64.

The minGRU-pytorch profile (intro; "Requirements & limits") describes the layer
as the log-space numerically stable version.  Written out, with
a_t = 1 - z_t and b_t = z_t g(p_t):

    log a_t = -softplus(k_t)
    log b_t = -softplus(-k_t) + log g(p_t)
    L_t     = sum_{s <= t} log a_s                     (cumulative sum)
    V_t     = L_t + logcumsumexp_{s <= t}(log b_s - L_s)
    h_t     = e^{L_t} h_0 + e^{V_t}

h_0 stays a linear term so that a signed carried state needs no logarithm.
This form is a check of the method (it must equal ``mingru.scan``), not the
parity target.

Also here: the pair (L, V) composition the parallel form is built from,
(L1, V1) (+) (L2, V2) = (L1 + L2, logaddexp(V1 + L2, V2)), with identity
(0, -inf).

Pinned by: agreement with the sequential definition to 1e-10 and the pair
composition's associativity (tests/test_oracle_mingru.py).
"""

from __future__ import annotations

import numpy as np

from . import scalar
from .mingru import _f64


def log_coefficients(k, p):
    """(log a, log b) = (-softplus(k), -softplus(-k) + log g(p))."""
    k = _f64(k)
    p = _f64(p)
    return -scalar.softplus(k), -scalar.softplus(-k) + scalar.log_g(p)


def scan(k, p, h0=None):
    la, lb = log_coefficients(k, p)
    L = np.cumsum(la, axis=1)
    V = L + np.logaddexp.accumulate(lb - L, axis=1)
    h = np.exp(V)
    if h0 is not None:
        h = h + np.exp(L) * _f64(h0)[:, None, :]
    return h


def pair_combine(first, second):
    """Compose two affine maps in log form: apply ``first`` then ``second``."""
    L1, V1 = first
    L2, V2 = second
    return L1 + L2, np.logaddexp(V1 + L2, V2)


PAIR_IDENTITY = (0.0, -np.inf)
