"""Oracle pins: the scalar activations against 50-digit mpmath and closed values."""

import numpy as np

from oracle import scalar
from tests import pins


def test_scalar_functions_match_mpmath():
    extra = np.random.default_rng(3).normal(0.0, 8.0, 64)
    err = pins.scalar_mp_err(scalar.sigmoid, scalar.softplus, scalar.g, scalar.log_g,
                             extra=extra)
    assert err < 4e-15, err


def test_scalar_special_values():
    assert pins.scalar_special_ok(scalar.sigmoid, scalar.softplus, scalar.g)


def test_g_is_continuous_at_zero():
    # Both branches give 1/2 at x = 0.
    eps = 1e-12
    assert abs(float(scalar.g(-eps)) - 0.5) < 1e-12
    assert abs(float(scalar.g(eps)) - 0.5) < 1e-12
    assert float(scalar.g(0.0)) == 0.5


def test_extreme_arguments_stay_finite():
    x = np.array([-1e4, -800.0, -100.0, 100.0, 800.0, 1e4])
    for f in (scalar.sigmoid, scalar.softplus, scalar.g):
        assert np.all(np.isfinite(f(x)))
    # log g at -1e4 is -1e4 (log sigma(x) ~ x for very negative x).
    assert abs(float(scalar.log_g(-1e4)) + 1e4) < 1e-9
