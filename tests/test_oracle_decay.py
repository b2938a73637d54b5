"""Pins of the time-decayed recurrence oracle, and planted mistakes that each
pin set must catch (all on the CPU, in oracle-side copies)."""

import numpy as np
import pytest

from oracle import decay, mingru, scalar
from tests import pins_decay as pd


def test_page_worked_example():
    assert pd.page_example_err(decay.scan, mingru.scan) == 0.0


def test_page_example_saturation_flags():
    """One saturated call with the raw gaps, none with log1p_delta, none for
    the zero-gap control."""
    _, _, lam = pd.page_case()
    gapped = np.array([pd.PAGE_GAPS])
    assert decay.saturated(lam, gapped)
    assert not decay.saturated(lam, gapped, log1p_delta=True)
    assert not decay.saturated(lam, np.zeros_like(gapped))
    # Only prefixes that reach the huge gap saturate.
    assert [decay.saturated(lam, gapped[:, :t]) for t in range(1, 7)] == \
        [False, False, False, True, True, True]


def test_no_decay_is_plain_mingru():
    assert pd.no_decay_err(decay.scan, mingru.scan) == 0.0


def test_closed_form_constant_inputs():
    assert pd.closed_const_err(decay.scan) < 1e-13


def test_rational_brute_force():
    assert pd.rational_err(decay.scan) < 1e-13


def test_log1p_reparameterisation():
    assert pd.log1p_err(decay.scan) < 1e-13


def test_clamp_threshold_and_wipe():
    lam = np.array([1.0, 2.0])
    at = np.array([[1.0e4 / 2.0]])          # 2 * 5000 = 1e4 exactly: not above
    assert not decay.saturated(lam, at)
    above = np.array([[np.nextafter(np.float32(5000.0), np.float32(1e9))]], dtype=np.float64)
    assert decay.saturated(lam, above)
    # A gap far past the clamp: gamma is exactly 0, no overflow, no NaN.
    e = decay.exponent(lam, np.array([[1e30]]))
    assert np.all(e == decay.SATURATION)
    assert np.all(decay.gamma(lam, np.array([[1e30]])) == 0.0)
    rng = np.random.default_rng(905)
    k = rng.normal(0, 1, (1, 5, 2))
    p = rng.normal(0, 1, (1, 5, 2))
    h0 = rng.normal(0, 1, (1, 2))
    dt = np.array([[1.0, 1e30, 1.0, 1.0, 1.0]])
    h = decay.scan(k, p, lam, dt, h0)
    fresh = decay.scan(k[:, 1:], p[:, 1:], lam, dt[:, 1:] * 0 + np.array([[0.0, 1, 1, 1]]))
    assert np.array_equal(h[:, 1:], fresh)


def test_carried_state_concatenation():
    rng = np.random.default_rng(906)
    B, T, D = 2, 50, 3
    k = rng.normal(0, 1, (B, T, D))
    p = rng.normal(0, 1, (B, T, D))
    lam = rng.uniform(0, 2, D)
    dt = rng.exponential(1.0, (B, T))
    h0 = rng.normal(0, 1, (B, D))
    full = decay.scan(k, p, lam, dt, h0)
    a = decay.scan(k[:, :17], p[:, :17], lam, dt[:, :17], h0)
    b = decay.scan(k[:, 17:], p[:, 17:], lam, dt[:, 17:], a[:, -1])
    assert np.array_equal(np.concatenate([a, b], axis=1), full)


def test_step_loop_matches_layer():
    rng = np.random.default_rng(907)
    B, T, D_in, D_h = 2, 12, 5, 4
    x = rng.normal(0, 1, (B, T, D_in))
    W_in = rng.normal(0, 0.5, (D_in, 2 * D_h))
    W_out = rng.normal(0, 0.5, (D_h, D_h))
    lam = rng.uniform(0, 2, D_h)
    dt = rng.exponential(1.0, (B, T))
    y, h, last = decay.layer(x, W_in, lam, dt, W_out, log1p_delta=True)
    hs = None
    for t in range(T):
        y_t, hs = decay.step(x[:, t], W_in, lam, dt[:, t], W_out, hs, log1p_delta=True)
        assert np.allclose(hs, h[:, t], rtol=1e-13, atol=0)
        assert np.allclose(y_t, y[:, t], rtol=1e-12, atol=1e-14)
    assert np.array_equal(last, h[:, -1])


def test_scan_terms_bound_h():
    rng = np.random.default_rng(908)
    k = rng.normal(0, 1, (2, 30, 4))
    p = rng.normal(0, 1, (2, 30, 4))
    lam = rng.uniform(0, 1, 4)
    dt = rng.exponential(1.0, (2, 30))
    h0 = rng.normal(0, 1, (2, 4))
    carry, inp = decay.scan_terms(k, p, lam, dt, h0)
    h = decay.scan(k, p, lam, dt, h0)
    assert np.all(np.abs(h) <= carry + inp + 1e-12)
    # With a non-negative h0 the two terms add up to h.
    h0p = np.abs(h0)
    carry, inp = decay.scan_terms(k, p, lam, dt, h0p)
    assert np.allclose(carry + inp, decay.scan(k, p, lam, dt, h0p), rtol=1e-13, atol=0)


# ------------------------------------------------------------ planted mistakes

def _decayed_scan(update):
    def scan(k, p, lam, dt, h0=None, log1p_delta=False):
        k = np.asarray(k, np.float64)
        p = np.asarray(p, np.float64)
        z = scalar.sigmoid(k)
        g = scalar.g(p)
        gam = decay.gamma(lam, dt, log1p_delta)
        B, T, D = k.shape
        h = np.zeros((B, D)) if h0 is None else np.asarray(h0, np.float64).copy()
        out = np.empty((B, T, D))
        for t in range(T):
            h = update(z, g, gam, h, t, T)
            out[:, t] = h
        return out
    return scan


decay_after_write = _decayed_scan(
    lambda z, g, gam, h, t, T: gam[:, t] * ((1 - z[:, t]) * h + z[:, t] * g[:, t]))
decay_next_gap = _decayed_scan(
    lambda z, g, gam, h, t, T: (1 - z[:, t]) * gam[:, min(t + 1, T - 1)] * h + z[:, t] * g[:, t])
decay_previous_gap = _decayed_scan(
    lambda z, g, gam, h, t, T: (1 - z[:, t]) * gam[:, max(t - 1, 0)] * h + z[:, t] * g[:, t])
decay_on_write_too = _decayed_scan(
    lambda z, g, gam, h, t, T: gam[:, t] * (1 - z[:, t]) * h + gam[:, t] * z[:, t] * g[:, t])
decay_dropped = _decayed_scan(
    lambda z, g, gam, h, t, T: (1 - z[:, t]) * h + z[:, t] * g[:, t])
decay_on_gate = _decayed_scan(   # decays the candidate's share instead of the state
    lambda z, g, gam, h, t, T: (1 - z[:, t] * gam[:, t]) * h + z[:, t] * gam[:, t] * g[:, t])


def decay_growth(k, p, lam, dt, h0=None, log1p_delta=False):
    return decay.scan(k, p, -np.asarray(lam, np.float64), dt, h0, log1p_delta)


def decay_transposed(k, p, lam, dt, h0=None, log1p_delta=False):
    """Rate indexed by batch row and gap by channel (only possible when the
    shapes happen to agree, as in the closed-form pin)."""
    k = np.asarray(k, np.float64)
    B, T, D = k.shape
    lam = np.asarray(lam, np.float64)
    dt = np.asarray(dt, np.float64)
    if lam.shape[0] != B or dt.shape[0] != D:
        return decay.scan(k, p, lam, dt, h0, log1p_delta)
    return decay.scan(k, p, dt[:, 0], lam[:, None] * np.ones((B, T)), h0, log1p_delta)


def decay_log_instead_of_log1p(k, p, lam, dt, h0=None, log1p_delta=False):
    if log1p_delta:
        with np.errstate(divide="ignore"):
            return decay.scan(k, p, lam, np.log(np.asarray(dt, np.float64)), h0)
    return decay.scan(k, p, lam, dt, h0)


@pytest.mark.parametrize("bad", [decay_after_write, decay_next_gap, decay_previous_gap,
                                 decay_on_write_too, decay_dropped, decay_on_gate,
                                 decay_growth, decay_transposed, decay_log_instead_of_log1p])
def test_pins_catch_planted_mistakes(bad):
    with np.errstate(all="ignore"):
        errs = [pd.page_example_err(bad, mingru.scan), pd.no_decay_err(bad, mingru.scan),
                pd.closed_const_err(bad), pd.rational_err(bad), pd.log1p_err(bad)]
    errs = [e if np.isfinite(e) else np.inf for e in errs]
    assert max(errs) > 1e-6, (bad.__name__, errs)
