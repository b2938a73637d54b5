"""Planted mistakes: each pin must fail on a copy of the oracle carrying a
plausible error (a dropped term, a wrong sign, a wrong index, a swapped
operand).  This is what makes the pins worth trusting.  Every mistake here is
planted in oracle-side code on the CPU."""

import numpy as np

from oracle import logspace, minmax, mingru, scalar
from tests import pins


# ------------------------------------------------------------ scalar mutants

def g_sigmoid_everywhere(x):
    return scalar.sigmoid(x)


def softplus_no_max(x):
    x = np.asarray(x, dtype=np.float64)
    return np.log1p(np.exp(-np.abs(x)))


def log_g_wrong_sign(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, np.log(np.maximum(x, 0) + 0.5), x + scalar.softplus(x))


def test_scalar_pins_catch_mistakes():
    good = pins.scalar_mp_err(scalar.sigmoid, scalar.softplus, scalar.g, scalar.log_g)
    assert good < 4e-15
    assert pins.scalar_mp_err(scalar.sigmoid, scalar.softplus, g_sigmoid_everywhere,
                              scalar.log_g) > 1e-3
    assert pins.scalar_mp_err(scalar.sigmoid, softplus_no_max, scalar.g, scalar.log_g) > 1e-3
    assert pins.scalar_mp_err(scalar.sigmoid, scalar.softplus, scalar.g,
                              log_g_wrong_sign) > 1e-3
    assert not pins.scalar_special_ok(scalar.sigmoid, scalar.softplus, g_sigmoid_everywhere)


# -------------------------------------------------------------- scan mutants

def _scan_with(update):
    def scan(k, p, h0=None):
        k = np.asarray(k, np.float64)
        p = np.asarray(p, np.float64)
        z = scalar.sigmoid(k)
        ht = scalar.g(p)
        B, T, D = k.shape
        h = np.zeros((B, D)) if h0 is None else np.asarray(h0, np.float64).copy()
        out = np.empty((B, T, D))
        for t in range(T):
            h = update(z, ht, h, t)
            out[:, t] = h
        return out
    return scan


scan_swapped_gate = _scan_with(lambda z, ht, h, t: z[:, t] * h + (1 - z[:, t]) * ht[:, t])
scan_candidate_off_by_one = _scan_with(
    lambda z, ht, h, t: (1 - z[:, t]) * h + z[:, t] * ht[:, max(t - 1, 0)])
scan_dropped_carry = _scan_with(lambda z, ht, h, t: z[:, t] * ht[:, t])
scan_gate_index_off = _scan_with(
    lambda z, ht, h, t: (1 - z[:, max(t - 1, 0)]) * h + z[:, t] * ht[:, t])


def scan_ignores_h0(k, p, h0=None):
    return mingru.scan(k, p, None)


def test_scan_pins_catch_mistakes():
    assert pins.scan_mp_err(mingru.scan) < 1e-14
    for bad in (scan_swapped_gate, scan_candidate_off_by_one, scan_dropped_carry,
                scan_gate_index_off, scan_ignores_h0):
        caught = (pins.scan_mp_err(bad) > 1e-6
                  or pins.closed_z1_err(bad, scalar.g) > 1e-6
                  or pins.closed_z0_err(bad) > 1e-6
                  or pins.closed_const_err(bad, scalar.sigmoid, scalar.g) > 1e-6
                  or pins.closed_conv_err(bad, scalar.sigmoid, scalar.g) > 1e-6)
        assert caught, bad
    # The closed forms alone already catch the gate and carry mistakes.
    assert pins.closed_z1_err(scan_swapped_gate, scalar.g) > 1e-3
    assert pins.closed_z0_err(scan_ignores_h0) > 1e-3
    assert pins.closed_z0_err(scan_dropped_carry) > 1e-3


def linear_wrong_order(a, b, h0=None):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    B, T, D = a.shape
    h = np.zeros((B, D)) if h0 is None else np.asarray(h0, np.float64).copy()
    out = np.empty((B, T, D))
    for t in range(T):
        h = a[:, t] * (h + b[:, t])
        out[:, t] = h
    return out


def test_linear_pin_catches_mistake():
    assert pins.linear_brute_err(mingru.linear_recurrence) < 1e-14
    assert pins.linear_brute_err(linear_wrong_order) > 1e-3


def logspace_wrong_sign(k, p, h0=None):
    k = np.asarray(k, np.float64)
    la = -scalar.softplus(k)
    lb = scalar.softplus(-k) + scalar.log_g(p)      # sign of log z flipped
    L = np.cumsum(la, axis=1)
    V = L + np.logaddexp.accumulate(lb - L, axis=1)
    h = np.exp(V)
    if h0 is not None:
        h = h + np.exp(L) * np.asarray(h0)[:, None, :]
    return h


def logspace_no_shift(k, p, h0=None):
    la, lb = logspace.log_coefficients(k, p)
    L = np.cumsum(la, axis=1)
    V = np.logaddexp.accumulate(lb, axis=1)         # dropped the -L / +L shift
    h = np.exp(V)
    if h0 is not None:
        h = h + np.exp(L) * np.asarray(h0)[:, None, :]
    return h


def test_logspace_pin_catches_mistakes():
    args = dict(T=512)
    assert pins.logspace_err(mingru.scan, logspace.scan, mingru.scan_terms, **args) < 1e-10
    assert pins.logspace_err(mingru.scan, logspace_wrong_sign, mingru.scan_terms, **args) > 1e-3
    assert pins.logspace_err(mingru.scan, logspace_no_shift, mingru.scan_terms, **args) > 1e-3


def logpair_dropped_shift(first, second):
    L1, V1 = first
    L2, V2 = second
    return L1 + L2, np.logaddexp(V1, V2)


def test_logpair_pin_catches_mistake():
    assert pins.logpair_groupings_err(logpair_dropped_shift) > 1e-3


# ------------------------------------------------------------ MinMax mutants

def _mm_scan_with(update, shift_output=False):
    def scan(r, s, x0):
        x = np.array(x0, copy=True)
        B, T, D = r.shape
        out = np.empty_like(r)
        for t in range(T):
            prev = x
            x = update(r[:, t], s[:, t], x)
            out[:, t] = prev if shift_output else x
        return out, x.copy()
    return scan


mm_swapped = _mm_scan_with(lambda r, s, x: np.minimum(np.maximum(r, x), s))
mm_off_by_one = _mm_scan_with(lambda r, s, x: np.maximum(np.minimum(r, x), s),
                              shift_output=True)
mm_no_floor = _mm_scan_with(lambda r, s, x: np.minimum(r, x))


def test_minmax_pins_catch_mistakes():
    for bad in (mm_swapped, mm_off_by_one, mm_no_floor):
        caught = not (pins.minmax_hold_ok(bad) and pins.minmax_reset_ok(bad)
                      and pins.minmax_brute_ok(bad) and pins.minmax_member_bound_ok(bad))
        assert caught, bad


def compose_wrong_floor(first, second):
    R1, S1 = first
    R2, S2 = second
    return np.minimum(R1, R2), np.maximum(S1, S2)


def compose_wrong_order(first, second):
    return minmax.compose(second, first)


def test_minmax_composition_pin_catches_mistakes():
    assert not pins.minmax_groupings_ok(compose_wrong_floor, minmax.apply, T=4)
    assert not pins.minmax_groupings_ok(compose_wrong_order, minmax.apply, T=4)
