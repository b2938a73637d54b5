"""Error measures used to compare a computed result with the oracle's.

* Hidden state h: |h - h_ref| / (|prod(1 - z)| |h_0| + h_ref(h_0 = 0)).  The
  denominator is the size of the two non-negative terms h is the sum of, so
  the measure stays meaningful where a signed h_0 makes h cross zero; it
  equals the plain relative error when h_0 >= 0 or is absent.
* Output y = h W_out: |y - y_ref| / (|h_ref| @ |W_out|), the componentwise
  condition bound of a dot product.
* MinMax: the float32 bit patterns must be equal.
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def h_rel_err(h, h_ref, carry_mag, input_term, floor=1e-300):
    """Max of the conditioned relative error of h (see module docstring)."""
    h = _f64(h)
    den = np.maximum(_f64(carry_mag) + _f64(input_term), floor)
    return float(np.max(np.abs(h - _f64(h_ref)) / den)) if h.size else 0.0


def y_rel_err(y, y_ref, h_ref, W_out, floor=1e-300):
    y = _f64(y)
    den = np.maximum(np.matmul(np.abs(_f64(h_ref)), np.abs(_f64(W_out))), floor)
    return float(np.max(np.abs(y - _f64(y_ref)) / den)) if y.size else 0.0


def max_abs_rel(a, ref):
    """max |a - ref| / max |ref| (a plain, unconditioned summary)."""
    a = _f64(a)
    ref = _f64(ref)
    if not a.size:
        return 0.0
    return float(np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1e-300))


def bits_equal(a, b) -> bool:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and bool(np.array_equal(a.view(np.uint32), b.view(np.uint32)))
