"""Oracle pins for the MinMax neuron's scan."""

import numpy as np
import pytest

from oracle import minmax
from tests import pins


def test_no_reset_holds_initial_state():
    assert pins.minmax_hold_ok(minmax.scan)


def test_single_forced_reset():
    assert pins.minmax_reset_ok(minmax.scan)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_membership_and_bounds(seed):
    assert pins.minmax_member_bound_ok(minmax.scan, seed=seed)


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_tiny(seed):
    assert pins.minmax_brute_ok(minmax.scan, seed=seed)


def test_grouping_enumeration_is_exhaustive():
    # Catalan numbers: 1, 1, 2, 5, 14, 42, 132
    assert [pins.all_groupings_count(n) for n in range(1, 8)] == [1, 1, 2, 5, 14, 42, 132]


@pytest.mark.parametrize("T", [2, 3, 5, 7])
def test_every_parenthesisation_of_the_composition(T):
    assert pins.minmax_groupings_ok(minmax.compose, minmax.apply, seed=T, T=T,
                                    trials=10 if T == 7 else 30)


def test_composition_random_pairs_bitwise():
    rng = np.random.default_rng(47)
    n = 200_000
    r1, r2 = rng.uniform(-1, 1, (2, n)).astype(np.float32)
    s1, s2 = (rng.uniform(-1, 1, (2, n)) - 0.5).astype(np.float32)
    x = rng.uniform(-1.5, 1.5, n).astype(np.float32)
    seq = minmax.apply((r2, s2), minmax.apply((r1, s1), x))
    comp = minmax.apply(minmax.compose((r1, s1), (r2, s2)), x)
    assert np.array_equal(seq.view(np.uint32), comp.view(np.uint32))


def test_identity_map():
    x = np.float32([-1.0, 0.0, 3.5])
    assert np.array_equal(minmax.apply(minmax.IDENTITY, x), x)
    m = (np.float32(0.25), np.float32(-0.5))
    assert minmax.compose(minmax.IDENTITY, m) == m
    assert minmax.compose(m, minmax.IDENTITY) == m


def test_float32_and_float64_give_the_same_bits():
    rng = np.random.default_rng(48)
    r = rng.uniform(-1, 1, (2, 500, 7)).astype(np.float32)
    s = (rng.uniform(-1, 1, (2, 500, 7)) - 0.5).astype(np.float32)
    x0 = rng.uniform(-1, 1, (2, 7)).astype(np.float32)
    o32, _ = minmax.scan(r, s, x0)
    o64, _ = minmax.scan(r.astype(np.float64), s.astype(np.float64), x0.astype(np.float64))
    assert np.array_equal(o32.view(np.uint32), o64.astype(np.float32).view(np.uint32))
