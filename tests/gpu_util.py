"""Helpers for the GPU parity tests: upload seeded inputs, run the oracle on
the same values, and report the conditioned errors."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import metrics, mingru

# The tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with fp32
# arithmetic (conditioned relative error, see oracle.metrics); MinMax is
# compared bit for bit.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(*args):
    """Print and flush, so a failing GPU run still names its case."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def host64(t):
    return t.detach().to("cpu").double().numpy()


def scan_err(h_gpu, k, p, h0):
    """Conditioned max relative error of h against the sequential oracle."""
    h_ref = mingru.scan(k, p, h0)
    carry, inp = mingru.scan_terms(k, p, h0)
    return metrics.h_rel_err(h_gpu, h_ref, carry, inp)
