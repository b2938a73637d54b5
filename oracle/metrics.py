"""Error measures used to compare a computed result with the oracle's.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages state no error measure; these are the readings of "max relative
error" that stay meaningful for this recurrence:

* Hidden state h: |h - h_ref| / (|prod(1 - z)| |h_0| + h_ref(h_0 = 0)).  The
  denominator is the size of the two non-negative terms h is the sum of, so
  the measure stays meaningful where a signed h_0 makes h cross zero; it
  equals the plain relative error when h_0 >= 0 or is absent.
* Output y = h W_out: |y - y_ref| / (|h_ref| @ |W_out|), the componentwise
  condition bound of a dot product.
* A plain summary, max |a - ref| / max |ref|.
* MinMax: the float32 bit patterns must be equal.

A result that is not finite where the reference is finite (a NaN or an
infinity produced by the computation) has error +inf, so that no tolerance
accepts it.

Pinned by hand-computed cases in tests/test_oracle_metrics.py (a signed
carried state crossing zero, a dot product with cancelling terms, NaN
results, +0 against -0, equal NaN payloads), each of which also fails a
planted mistake (the minimum instead of the maximum, a denominator without
the carry term or without |W_out|, a float instead of a bit compare, NaN
skipped).
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _nonfinite_where_ref_finite(x, ref) -> bool:
    return bool(np.any(~np.isfinite(x) & np.isfinite(ref)))


def h_rel_err(h, h_ref, carry_mag, input_term, floor=1e-300):
    """Max of the conditioned relative error of h (see module docstring)."""
    h = _f64(h)
    h_ref = _f64(h_ref)
    if not h.size:
        return 0.0
    if _nonfinite_where_ref_finite(h, h_ref):
        return float("inf")
    den = np.maximum(_f64(carry_mag) + _f64(input_term), floor)
    return float(np.max(np.abs(h - h_ref) / den))


def y_rel_err(y, y_ref, h_ref, W_out, floor=1e-300):
    """Max of |y - y_ref| / (|h_ref| @ |W_out|) (see module docstring)."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    if not y.size:
        return 0.0
    if _nonfinite_where_ref_finite(y, y_ref):
        return float("inf")
    den = np.maximum(np.matmul(np.abs(_f64(h_ref)), np.abs(_f64(W_out))), floor)
    return float(np.max(np.abs(y - y_ref) / den))


def max_abs_rel(a, ref):
    """max |a - ref| / max |ref| (a plain, unconditioned summary)."""
    a = _f64(a)
    ref = _f64(ref)
    if not a.size:
        return 0.0
    if _nonfinite_where_ref_finite(a, ref):
        return float("inf")
    return float(np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _f32_array(x, name):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError(f"bits_equal compares float32 bit patterns; {name} is {x.dtype}")
    return np.ascontiguousarray(x)


def bits_equal(a, b) -> bool:
    """True when a and b (both float32) have the same shape and bit patterns."""
    a = _f32_array(a, "a")
    b = _f32_array(b, "b")
    return a.shape == b.shape and bool(np.array_equal(a.view(np.uint32), b.view(np.uint32)))
