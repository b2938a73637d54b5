"""The MinMax neuron's recurrence, run sequentially.

minmaxrnc PyPI page, "The model" item 3: the hidden state is updated element
by element as x_{t+1} = max(min(r_t, x_t), s_t), and the whole sequence is
computed in parallel by a prefix scan ("Key properties": O(log T) depth).

Readings: the inputs r, s have T steps and the output holds x_1 .. x_T (x_0,
the carried state, is not repeated in the output); x_0 is required.  min and
max only select one of their operands, so running this in float32 or float64
gives the same bits.

Also here: the clamp-composition rule a prefix scan over this update needs.
Applying (R1, S1) then (R2, S2) to x gives
    max(min(R2, max(min(R1, x), S1)), S2)
  = max(min(min(R1, R2), x), max(min(R2, S1), S2))
by distributivity of min over max on a total order, so the composed map is
again a clamp (min(R1, R2), max(min(R2, S1), S2)); the identity is
(+inf, -inf).

Pinned by: closed forms (no reset keeps x_0; a single forced reset), the
membership and boundedness invariants, and an exhaustive check that every
parenthesisation of the composition gives the sequential result bit for bit
(tests/test_oracle_minmax.py).
"""

from __future__ import annotations

import numpy as np


def scan(r, s, x0):
    """x_out[:, t] = x_{t+1}; returns (x_out [B,T,D], x_last [B,D]) in r's dtype."""
    r = np.asarray(r)
    s = np.asarray(s)
    x = np.array(x0, dtype=r.dtype, copy=True)
    B, T, D = r.shape
    out = np.empty((B, T, D), dtype=r.dtype)
    for t in range(T):
        x = np.maximum(np.minimum(r[:, t, :], x), s[:, t, :])
        out[:, t, :] = x
    return out, x.copy()


def apply(rs, x):
    """Apply one clamp map (R, S) to x."""
    R, S = rs
    return np.maximum(np.minimum(R, x), S)


def compose(first, second):
    """The clamp map equal to applying ``first`` then ``second``."""
    R1, S1 = first
    R2, S2 = second
    return np.minimum(R1, R2), np.maximum(np.minimum(R2, S1), S2)


IDENTITY = (np.inf, -np.inf)
