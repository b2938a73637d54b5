"""Fits the polynomial the scans use for 1 - 2^y at small y <= 0 (the
complement of a time-decay factor, see decay_factors in scan_engine.hpp) and
checks it in fp32 arithmetic as the kernels evaluate it.

    python scan_linear_rnn_amd/csrc/decay_poly.py

Q(y) = (1 - 2^y) / y on [-log2(e)/8, 0] (x = -y ln 2 in [0, 1/8]) is fitted
with a cubic by iteratively reweighted least squares on Chebyshev nodes
(relative error, towards minimax); 1 - 2^y = y Q(y) then has no cancelling
subtraction.  The fp32 evaluation (Horner with fused multiply-adds, then
times y) is compared with 1 - 2^y in 40-digit arithmetic.
"""
import mpmath as mp
import numpy as np

mp.mp.dps = 40
Y_LO = -0.125 / np.log(2.0)
DEG = 3


def q_exact(y):
    y = mp.mpf(y)
    return -mp.log(2) if y == 0 else (1 - mp.power(2, y)) / y


def fit():
    n = 400
    ys = Y_LO / 2 + (Y_LO / 2) * np.cos(np.pi * (np.arange(n) + 0.5) / n)
    qv = np.array([float(q_exact(y)) for y in ys])
    V = np.vander(ys, DEG + 1, increasing=True)
    w = 1.0 / np.abs(qv)
    coef, *_ = np.linalg.lstsq(V * w[:, None], qv * w, rcond=None)
    for _ in range(50):
        r = (V @ coef - qv) / qv
        w2 = w * np.sqrt(np.abs(r) / np.abs(r).max() + 1e-3)
        coef, *_ = np.linalg.lstsq(V * w2[:, None], qv * w2, rcond=None)
    return coef.astype(np.float32)


def fp32_complement(c, y32):
    q = np.full_like(y32, c[DEG])
    for k in range(DEG - 1, -1, -1):  # fma: exact product and sum, one rounding
        q = (q.astype(np.float64) * y32.astype(np.float64) + np.float64(c[k])).astype(np.float32)
    return (q.astype(np.float64) * y32.astype(np.float64)).astype(np.float32)


if __name__ == "__main__":
    c = fit()
    print("coefficients (y^0 .. y^3):", ", ".join(f"{float(v):.9g}f" for v in c))
    y32 = np.linspace(Y_LO, 0.0, 40001)[:-1].astype(np.float32)
    om = fp32_complement(c, y32)
    ref = np.array([float(1 - mp.power(2, mp.mpf(float(v)))) for v in y32])
    print("max relative error in fp32:", float(np.max(np.abs(om - ref) / ref)))
