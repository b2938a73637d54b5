"""Pins for the error measures every parity test is judged by (oracle.metrics).

Each case is small enough to work out by hand; the expected numbers are
written as exact binary fractions.  Each pin takes the measure under test as
an argument, so the same pin runs against a copy of the measure carrying a
plausible mistake, which must fail it (planted on the CPU, in copies here).
"""

import math

import numpy as np
import pytest
import torch

from oracle import metrics

# ----------------------------------------------------------------------- h
#
# A signed carried state crossing zero: h = -carry + input with carry =
# |prod(1 - z)| |h_0| (h_0 < 0) and input the zero-state response.
#   h_ref  = [-0.25, 2^-7, 0.5]
#   carry  = [0.75, 0.5 - 2^-7, 0.25]
#   input  = [0.5, 0.5, 0.75]          (input - carry = h_ref)
#   h      = h_ref + [2^-20, 2^-20, -2^-19]
# Conditioned: 2^-20/1.25, 2^-20/0.9921875, 2^-19/1  ->  max = 2^-19.
# The plain relative error at the middle element is 2^-20 / 2^-7 = 2^-13
# (above a 1e-4 bar); the conditioned one is far below it.
H_REF = np.array([-0.25, 2.0 ** -7, 0.5])
CARRY = np.array([0.75, 0.5 - 2.0 ** -7, 0.25])
INPUT = np.array([0.5, 0.5, 0.75])
H_ERR = np.array([2.0 ** -20, 2.0 ** -20, -(2.0 ** -19)])


def h_pin_ok(h_rel_err) -> bool:
    assert np.array_equal(INPUT - CARRY, H_REF)
    got = h_rel_err(H_REF + H_ERR, H_REF, CARRY, INPUT)
    if got != 2.0 ** -19:
        return False
    # Exact results have zero error; a NaN or infinite result never passes.
    if h_rel_err(H_REF, H_REF, CARRY, INPUT) != 0.0:
        return False
    bad = (H_REF + H_ERR).copy()
    bad[1] = np.nan
    e = h_rel_err(bad, H_REF, CARRY, INPUT)
    if not (e == math.inf):
        return False
    bad[1] = np.inf
    return h_rel_err(bad, H_REF, CARRY, INPUT) == math.inf


# ----------------------------------------------------------------------- y
#
# One row, D_h = 2, D_out = 2:
#   h_ref = [1, -2],  W_out = [[1, 2], [1, -1]]
#   y_ref = h_ref W_out = [-1, 4],  |h_ref| |W_out| = [3, 4]
#   y     = y_ref + [3 * 2^-20, 2^-20]
# Conditioned: 2^-20, 2^-22  ->  max = 2^-20.  The absolute values matter:
# |h_ref| with a signed W_out gives the second denominator 1*2 + 2*(-1) = 0,
# and a signed h_ref with |W_out| gives the first 1*1 + (-2)*1 = -1.
Y_H = np.array([[[1.0, -2.0]]])
Y_W = np.array([[1.0, 2.0], [1.0, -1.0]])
Y_REF = np.array([[[-1.0, 4.0]]])
Y_ERR = np.array([[[3 * 2.0 ** -20, 2.0 ** -20]]])


def y_pin_ok(y_rel_err) -> bool:
    assert np.array_equal(np.matmul(Y_H, Y_W), Y_REF)
    if y_rel_err(Y_REF + Y_ERR, Y_REF, Y_H, Y_W) != 2.0 ** -20:
        return False
    bad = Y_REF.copy()
    bad[0, 0, 1] = np.nan
    return y_rel_err(bad, Y_REF, Y_H, Y_W) == math.inf


# ------------------------------------------------------------ max_abs_rel
#
#   ref = [1, -4, 2],  a = [1, -4 - 2^-9, 2]
#   max |a - ref| = 2^-9,  max |ref| = 4  ->  2^-11
# (max |a| = 4 + 2^-9 would give a different value).
M_REF = np.array([1.0, -4.0, 2.0])
M_A = np.array([1.0, -4.0 - 2.0 ** -9, 2.0])


def maxabs_pin_ok(max_abs_rel) -> bool:
    if max_abs_rel(M_A, M_REF) != 2.0 ** -11:
        return False
    bad = M_A.copy()
    bad[0] = np.nan
    return max_abs_rel(bad, M_REF) == math.inf


# -------------------------------------------------------------- bits_equal

def bits_pin_ok(bits_equal) -> bool:
    one = np.array([1.0, -2.5, 3.0e-38], np.float32)
    if not bits_equal(one, one.copy()):
        return False
    # +0 and -0 are equal as numbers but not as bits.
    if bits_equal(np.array([0.0], np.float32), np.array([-0.0], np.float32)):
        return False
    # The same NaN payload is the same bits (a float compare says unequal).
    nan = np.array([np.nan], np.float32)
    if not bits_equal(nan, nan.copy()):
        return False
    # One unit in the last place apart.
    nxt = np.nextafter(one, np.float32(np.inf), dtype=np.float32)
    if bits_equal(one, nxt):
        return False
    # Shapes must agree.
    if bits_equal(one, one[:2]):
        return False
    # Torch tensors are read as their float32 values.
    return bits_equal(torch.from_numpy(one), one)


def test_h_rel_err_hand_computed():
    assert h_pin_ok(metrics.h_rel_err)
    plain = np.max(np.abs(H_ERR) / np.abs(H_REF))
    assert plain > 1e-4 > metrics.h_rel_err(H_REF + H_ERR, H_REF, CARRY, INPUT)


def test_y_rel_err_hand_computed():
    assert y_pin_ok(metrics.y_rel_err)


def test_max_abs_rel_hand_computed():
    assert maxabs_pin_ok(metrics.max_abs_rel)


def test_bits_equal_cases():
    assert bits_pin_ok(metrics.bits_equal)


def test_bits_equal_refuses_other_dtypes():
    # A float64 array rounded to float32 could compare equal after rounding.
    with pytest.raises(TypeError):
        metrics.bits_equal(np.array([1.0 + 1e-12]), np.array([1.0], np.float32))


def test_empty_inputs_have_zero_error():
    e = np.zeros((0, 3))
    assert metrics.h_rel_err(e, e, e, e) == 0.0
    assert metrics.max_abs_rel(e, e) == 0.0


# ------------------------------------------------------- planted mistakes

def h_min_instead_of_max(h, h_ref, carry_mag, input_term, floor=1e-300):
    h = np.asarray(h, np.float64)
    den = np.maximum(carry_mag + input_term, floor)
    return float(np.min(np.abs(h - h_ref) / den))


def h_without_carry(h, h_ref, carry_mag, input_term, floor=1e-300):
    h = np.asarray(h, np.float64)
    if np.any(~np.isfinite(h)):
        return math.inf
    den = np.maximum(input_term, floor)
    return float(np.max(np.abs(h - h_ref) / den))


def h_nan_skipped(h, h_ref, carry_mag, input_term, floor=1e-300):
    h = np.asarray(h, np.float64)
    den = np.maximum(carry_mag + input_term, floor)
    return float(np.nanmax(np.abs(h - h_ref) / den))


def h_plain_relative(h, h_ref, carry_mag, input_term, floor=1e-300):
    h = np.asarray(h, np.float64)
    if np.any(~np.isfinite(h)):
        return math.inf
    return float(np.max(np.abs(h - h_ref) / np.maximum(np.abs(h_ref), floor)))


def y_signed_w(y, y_ref, h_ref, W_out, floor=1e-300):
    y = np.asarray(y, np.float64)
    if np.any(~np.isfinite(y)):
        return math.inf
    den = np.maximum(np.matmul(np.abs(h_ref), W_out), floor)
    return float(np.max(np.abs(y - y_ref) / den))


def y_signed_h(y, y_ref, h_ref, W_out, floor=1e-300):
    y = np.asarray(y, np.float64)
    if np.any(~np.isfinite(y)):
        return math.inf
    den = np.maximum(np.matmul(h_ref, np.abs(W_out)), floor)
    return float(np.max(np.abs(y - y_ref) / den))


def maxabs_over_a(a, ref):
    a = np.asarray(a, np.float64)
    if np.any(~np.isfinite(a)):
        return math.inf
    return float(np.max(np.abs(a - ref)) / np.max(np.abs(a)))


def maxabs_mean(a, ref):
    a = np.asarray(a, np.float64)
    return float(np.mean(np.abs(a - ref)) / np.max(np.abs(ref)))


def bits_as_float64(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return a.shape == b.shape and bool(np.array_equal(a, b))


def bits_after_cast(a, b):
    a = np.ascontiguousarray(np.asarray(a), dtype=np.float32)
    b = np.ascontiguousarray(np.asarray(b), dtype=np.float32)
    return a.shape == b.shape and bool(np.array_equal(a.view(np.uint32), b.view(np.uint32)))


@pytest.mark.parametrize("bad", [h_min_instead_of_max, h_without_carry, h_nan_skipped,
                                 h_plain_relative])
def test_h_pin_catches(bad):
    assert not h_pin_ok(bad)


@pytest.mark.parametrize("bad", [y_signed_w, y_signed_h])
def test_y_pin_catches(bad):
    assert not y_pin_ok(bad)


@pytest.mark.parametrize("bad", [maxabs_over_a, maxabs_mean])
def test_maxabs_pin_catches(bad):
    assert not maxabs_pin_ok(bad)


def test_bits_pin_catches_float_compare():
    assert not bits_pin_ok(bits_as_float64)


def test_bits_dtype_check_catches_silent_cast():
    # The rounding cast makes a float64 value off by 1e-12 compare equal.
    assert bits_after_cast(np.array([1.0 + 1e-12]), np.array([1.0], np.float32))
    with pytest.raises(TypeError):
        metrics.bits_equal(np.array([1.0 + 1e-12]), np.array([1.0], np.float32))
