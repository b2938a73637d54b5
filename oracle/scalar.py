"""Scalar activations of the minGRU cell, float64, element-wise.

Definitions (the method as stated for the minGRU profile's log-space layer,
minGRU-pytorch profile, intro and "Requirements & limits"):

    sigma(x)    = 1 / (1 + e^-x)
    softplus(x) = log(1 + e^x)
    g(x)        = x + 1/2          for x >= 0
                = sigma(x)         for x <  0
    log g(x)    = log(x + 1/2)     for x >= 0
                = x - softplus(x)  for x <  0      (log sigma(x))

At x = 0 both branches of g give 1/2, so g is continuous (reading: the x >= 0
branch owns x = 0).

Pinned by: 50-digit mpmath values on a grid and closed special values
(tests/test_oracle_scalar.py).
"""

from __future__ import annotations

import numpy as np


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    # Two algebraically equal forms, each used where e^(-|x|) cannot overflow.
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def g(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, x + 0.5, sigmoid(x))


def log_g(x):
    x = np.asarray(x, dtype=np.float64)
    pos = np.log(np.maximum(x, 0.0) + 0.5)
    neg = x - softplus(x)
    return np.where(x >= 0, pos, neg)
