"""Oracle pins for the minGRU recurrence, its layer and its step."""

import math

import numpy as np
import pytest

from oracle import logspace, mingru, scalar
from tests import pins


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_linear_recurrence_exact_rational(seed):
    assert pins.linear_brute_err(mingru.linear_recurrence, seed=seed) < 1e-14


@pytest.mark.parametrize("seed,with_h0,k_mean", [(0, True, 0.0), (1, False, 0.0),
                                                 (2, True, -3.0), (3, True, 3.0)])
def test_scan_against_mpmath_unrolled_sum(seed, with_h0, k_mean):
    err = pins.scan_mp_err(mingru.scan, seed=seed, with_h0=with_h0, k_mean=k_mean)
    assert err < 1e-14, err


def test_closed_form_z_one():
    assert pins.closed_z1_err(mingru.scan, scalar.g) == 0.0


def test_closed_form_z_zero():
    assert pins.closed_z0_err(mingru.scan) < 1e-15


def test_closed_form_constant_gate_constant_candidate():
    assert pins.closed_const_err(mingru.scan, scalar.sigmoid, scalar.g) < 1e-13


def test_closed_form_constant_gate_convolution():
    assert pins.closed_conv_err(mingru.scan, scalar.sigmoid, scalar.g) < 1e-12


@pytest.mark.parametrize("k_mean,with_h0", [(-4.0, True), (0.0, False), (2.0, True)])
def test_log_space_form_equals_sequential(k_mean, with_h0):
    err = pins.logspace_err(mingru.scan, logspace.scan, mingru.scan_terms,
                            k_mean=k_mean, with_h0=with_h0)
    assert err < 1e-10, err


def test_log_pair_composition_is_associative_and_affine():
    for seed in range(4):
        assert pins.logpair_groupings_err(logspace.pair_combine, seed=seed) < 1e-12


def test_log_pair_identity_has_no_nan():
    L, V = logspace.pair_combine(logspace.PAIR_IDENTITY, logspace.PAIR_IDENTITY)
    assert L == 0.0 and V == -np.inf
    L, V = logspace.pair_combine(logspace.PAIR_IDENTITY, (-0.5, 0.25))
    assert L == -0.5 and V == 0.25


def test_scan_terms_decompose_h():
    rng = np.random.default_rng(5)
    k = rng.normal(-1.0, 1.0, (2, 100, 3))
    p = rng.normal(0.0, 1.0, (2, 100, 3))
    h0 = rng.normal(0.0, 1.0, (2, 3))
    h = mingru.scan(k, p, h0)
    carry, inp = mingru.scan_terms(k, p, h0)
    # h = sign(h0) * carry + input_term, and |h| <= carry + input_term.
    assert np.max(np.abs(h - (np.sign(h0)[:, None, :] * carry + inp))) < 1e-13
    assert np.all(np.abs(h) <= carry + inp + 1e-13)


def test_convex_hull_and_positivity_invariants():
    rng = np.random.default_rng(6)
    k = rng.normal(0.0, 2.0, (2, 200, 4))
    p = rng.normal(0.0, 2.0, (2, 200, 4))
    h0 = rng.uniform(0.0, 2.0, (2, 4))
    h = mingru.scan(k, p, h0)
    ht = scalar.g(p)
    lo = np.minimum.accumulate(np.concatenate([h0[:, None, :], ht], axis=1), axis=1)[:, 1:]
    hi = np.maximum.accumulate(np.concatenate([h0[:, None, :], ht], axis=1), axis=1)[:, 1:]
    assert np.all(h >= lo - 1e-14) and np.all(h <= hi + 1e-14)
    assert np.all(mingru.scan(k, p, None) > 0)


def test_projection_dot_product_and_kp_columns():
    rng = np.random.default_rng(8)
    x = rng.normal(0.0, 1.0, (1, 3, 5))
    W = rng.normal(0.0, 1.0, (5, 6))
    kp = mingru.project(x, W)
    for t in range(3):
        for j in range(6):
            ref = math.fsum(x[0, t, i] * W[i, j] for i in range(5))
            assert abs(kp[0, t, j] - ref) < 1e-14
    # k is the first half of the columns: drive it to +40 so z = 1 and h = g(p).
    D_h = 3
    W2 = np.zeros((2, 2 * D_h))
    W2[0, :D_h] = 40.0          # k = 40 * x0 (x0 = 1)
    W2[1, D_h:] = 1.0           # p = x1
    xx = np.stack([np.ones(7), np.linspace(-2, 2, 7)], axis=-1)[None]
    y, h, _ = mingru.layer(xx, W2)
    assert np.array_equal(h, np.broadcast_to(scalar.g(xx[..., 1:2]), h.shape))


def test_carried_state_concatenation():
    rng = np.random.default_rng(9)
    x = rng.normal(0.0, 1.0, (2, 40, 6))
    W_in = rng.normal(0.0, 6 ** -0.5, (6, 8))
    W_out = rng.normal(0.0, 4 ** -0.5, (4, 5))
    y, h, last = mingru.layer(x, W_in, W_out)
    y1, h1, last1 = mingru.layer(x[:, :17], W_in, W_out)
    y2, h2, last2 = mingru.layer(x[:, 17:], W_in, W_out, h0=last1)
    assert np.allclose(np.concatenate([y1, y2], axis=1), y, rtol=0, atol=1e-14)
    assert np.allclose(last2, last, rtol=0, atol=1e-14)


def test_step_loop_equals_parallel_layer():
    rng = np.random.default_rng(10)
    x = rng.normal(0.0, 1.0, (3, 25, 4))
    W_in = rng.normal(0.0, 0.5, (4, 6))
    W_out = rng.normal(0.0, 0.5, (3, 3))
    y, h, last = mingru.layer(x, W_in, W_out)
    hp = None
    for t in range(25):
        yt, hp = mingru.step(x[:, t], W_in, W_out, hp)
        assert np.allclose(yt, y[:, t], rtol=0, atol=1e-14)
    assert np.allclose(hp, last, rtol=0, atol=1e-14)
