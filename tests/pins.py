"""Pins for the oracle: checks against things other than the oracle itself.

Each pin takes the function(s) under test as arguments and returns an error
measure (or a bool), so the same pin runs against the oracle and against
copies of it with a mistake planted (tests/test_oracle_mutations.py), which
shows that each plausible mistake is caught.

What pins what:
* scalar functions      -- 50-digit mpmath and closed special values;
* linear recurrence     -- exact rational brute force of the unrolled sum;
* minGRU scan           -- 40-digit mpmath of the unrolled sum from (k, p);
                           closed forms for z = 1, z = 0, constant z;
* log-space form        -- agreement with the sequential definition;
* MinMax                -- closed forms, membership / bounds, and every
                           parenthesisation of the clamp composition.
"""

from __future__ import annotations

from fractions import Fraction

import mpmath
import numpy as np

SCALAR_GRID = np.array([-40.0, -30.0, -12.5, -4.0, -1.0, -0.3, -1e-8, 0.0, 1e-8,
                        0.3, 0.5, 1.0, 2.0, 4.0, 12.5, 30.0, 40.0])


def _mp_sigmoid(x):
    return 1 / (1 + mpmath.exp(-x))


def _mp_softplus(x):
    return mpmath.log(1 + mpmath.exp(x))


def _mp_g(x):
    return x + mpmath.mpf("0.5") if x >= 0 else _mp_sigmoid(x)


def scalar_mp_err(sigmoid, softplus, g, log_g, extra=()) -> float:
    """Max relative error of the four scalar functions against mpmath."""
    mpmath.mp.dps = 50
    xs = np.concatenate([SCALAR_GRID, np.asarray(extra, dtype=np.float64)])
    worst = 0.0
    for x in xs:
        xm = mpmath.mpf(float(x))
        refs = {
            "sigmoid": _mp_sigmoid(xm),
            "softplus": _mp_softplus(xm),
            "g": _mp_g(xm),
            "log_g": mpmath.log(_mp_g(xm)),
            # log(1 - sigma(k)) = -softplus(k): the log-space coefficient.
            "log1m_sigmoid": mpmath.log(1 - _mp_sigmoid(xm)),
        }
        got = {
            "sigmoid": float(sigmoid(x)),
            "softplus": float(softplus(x)),
            "g": float(g(x)),
            "log_g": float(log_g(x)),
            "log1m_sigmoid": -float(softplus(x)),
        }
        for key, ref in refs.items():
            if ref == 0:
                err = abs(got[key])
            else:
                err = float(abs((mpmath.mpf(got[key]) - ref) / ref))
            worst = max(worst, err)
    return worst


def scalar_special_ok(sigmoid, softplus, g) -> bool:
    return (float(g(0.0)) == 0.5 and float(g(1.0)) == 1.5 and float(g(2.5)) == 3.0
            and float(sigmoid(0.0)) == 0.5
            and abs(float(softplus(0.0)) - np.log(2.0)) < 1e-16
            and abs(float(g(-1.0)) - 1.0 / (1.0 + np.e)) < 1e-16)


def linear_brute_err(linear_recurrence, seed=0, T=10, D=3) -> float:
    """Exact rational h_t = (prod a) h_0 + sum_s b_s prod_{r>s} a_r."""
    rng = np.random.default_rng([7, seed])
    a = rng.uniform(0.05, 0.99, (1, T, D))
    b = rng.normal(0.0, 1.0, (1, T, D))
    h0 = rng.normal(0.0, 1.0, (1, D))
    got = linear_recurrence(a, b, h0)
    worst = 0.0
    for d in range(D):
        A = [Fraction(float(v)) for v in a[0, :, d]]
        Bv = [Fraction(float(v)) for v in b[0, :, d]]
        H0 = Fraction(float(h0[0, d]))
        for t in range(T):
            prod_all = Fraction(1)
            for r in range(t + 1):
                prod_all *= A[r]
            total = prod_all * H0
            scale = abs(prod_all * H0)
            for s in range(t + 1):
                pr = Fraction(1)
                for r in range(s + 1, t + 1):
                    pr *= A[r]
                total += Bv[s] * pr
                scale += abs(Bv[s] * pr)
            err = abs(Fraction(float(got[0, t, d])) - total) / scale
            worst = max(worst, float(err))
    return worst


def scan_mp_err(scan, seed=0, T=12, D=3, with_h0=True, k_mean=0.0) -> float:
    """40-digit mpmath of the unrolled minGRU sum from the same (k, p)."""
    mpmath.mp.dps = 40
    rng = np.random.default_rng([11, seed])
    k = rng.normal(k_mean, 2.0, (1, T, D))
    p = rng.normal(0.0, 2.0, (1, T, D))
    h0 = rng.normal(0.0, 1.0, (1, D)) if with_h0 else None
    got = scan(k, p, h0)
    worst = 0.0
    for d in range(D):
        z = [_mp_sigmoid(mpmath.mpf(float(v))) for v in k[0, :, d]]
        ht = [_mp_g(mpmath.mpf(float(v))) for v in p[0, :, d]]
        H0 = mpmath.mpf(float(h0[0, d])) if with_h0 else mpmath.mpf(0)
        for t in range(T):
            dec = mpmath.mpf(1)
            for r in range(t + 1):
                dec *= 1 - z[r]
            total = dec * H0
            scale = abs(dec * H0)
            for s in range(t + 1):
                pr = mpmath.mpf(1)
                for r in range(s + 1, t + 1):
                    pr *= 1 - z[r]
                total += z[s] * ht[s] * pr
                scale += abs(z[s] * ht[s] * pr)
            worst = max(worst, float(abs(mpmath.mpf(float(got[0, t, d])) - total) / scale))
    return worst


def closed_z1_err(scan, g) -> float:
    """k = +800: sigma(k) is exactly 1 and sigma(-k) exactly 0 in float64
    (e^-800 underflows), so h_t = g(p_t)."""
    rng = np.random.default_rng(21)
    p = rng.normal(0.0, 3.0, (2, 50, 4))
    k = np.full_like(p, 800.0)
    h0 = rng.normal(0.0, 1.0, (2, 4))
    h = scan(k, p, h0)
    return float(np.max(np.abs(h - g(p))))


def closed_z0_err(scan) -> float:
    """k = -40: z = 4.2e-18, so h_t = h_0 to within 1e-15 over 200 steps."""
    rng = np.random.default_rng(22)
    p = rng.normal(0.0, 3.0, (2, 200, 4))
    k = np.full_like(p, -40.0)
    h0 = rng.normal(0.0, 1.0, (2, 4))
    h = scan(k, p, h0)
    return float(np.max(np.abs(h - h0[:, None, :])))


def closed_const_err(scan, sigmoid, g) -> float:
    """Constant z = c and constant candidate u: h_t = u + (1 - c)^t (h_0 - u)."""
    T = 300
    kval, pval = -1.3, 0.7
    k = np.full((1, T, 2), kval)
    p = np.full((1, T, 2), pval)
    h0 = np.array([[2.0, -3.0]])
    c = float(sigmoid(kval))
    u = float(g(pval))
    t = np.arange(1, T + 1)[None, :, None]
    ref = u + (1.0 - c) ** t * (h0[:, None, :] - u)
    return float(np.max(np.abs(scan(k, p, h0) - ref)))


def closed_conv_err(scan, sigmoid, g) -> float:
    """Constant z = c, varying candidate: h_t = (1-c)^t h_0 + c sum_s (1-c)^(t-s) g(p_s),
    the sum evaluated as a discrete convolution."""
    T = 256
    rng = np.random.default_rng(23)
    kval = 0.4
    p = rng.normal(0.0, 2.0, (1, T, 1))
    k = np.full_like(p, kval)
    h0 = np.array([[1.5]])
    c = float(sigmoid(kval))
    ht = g(p[0, :, 0])
    kern = (1.0 - c) ** np.arange(T)
    conv = np.convolve(ht, kern)[:T]
    t = np.arange(1, T + 1)
    ref = (1.0 - c) ** t * h0[0, 0] + c * conv
    return float(np.max(np.abs(scan(k, p, h0)[0, :, 0] - ref)))


def logspace_err(seq_scan, log_scan, carry_terms, seed=0, B=2, T=4096, D=8,
                 k_mean=-4.0, with_h0=True) -> float:
    """The log-space parallel form against the sequential form (conditioned)."""
    rng = np.random.default_rng([31, seed])
    k = rng.normal(k_mean, 1.0, (B, T, D))
    p = rng.normal(0.0, 1.0, (B, T, D))
    h0 = rng.normal(0.0, 1.0, (B, D)) if with_h0 else None
    hs = seq_scan(k, p, h0)
    hl = log_scan(k, p, h0)
    cm, it = carry_terms(k, p, h0)
    return float(np.max(np.abs(hs - hl) / (cm + it)))


# ---------------------------------------------------------------- MinMax

def minmax_hold_ok(scan) -> bool:
    """r = +2, s = -2 with x_0 in (-1, 1): no step can change x, x_t = x_0."""
    rng = np.random.default_rng(41)
    B, T, D = 2, 300, 5
    r = np.full((B, T, D), 2.0, np.float32)
    s = np.full((B, T, D), -2.0, np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    out, last = scan(r, s, x0)
    return bool(np.array_equal(out, np.broadcast_to(x0[:, None, :], out.shape))
                and np.array_equal(last, x0))


def minmax_reset_ok(scan) -> bool:
    """One forced reset at t*: r_{t*} = -3 < s_{t*} = v, so x_t = v after it."""
    rng = np.random.default_rng(42)
    B, T, D = 2, 300, 5
    r = np.full((B, T, D), 2.0, np.float32)
    s = np.full((B, T, D), -2.0, np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    tstar = 137
    v = rng.uniform(-1.5, 1.5, (B, D)).astype(np.float32)
    r[:, tstar, :] = -3.0
    s[:, tstar, :] = v
    out, _ = scan(r, s, x0)
    before = np.array_equal(out[:, :tstar], np.broadcast_to(x0[:, None, :], (B, tstar, D)))
    after = np.array_equal(out[:, tstar:], np.broadcast_to(v[:, None, :], (B, T - tstar, D)))
    return bool(before and after)


def minmax_member_bound_ok(scan, seed=0) -> bool:
    """Every output is bitwise one of {x_0, r_., s_.} of its channel, and lies
    between the channel's smallest and largest input (the operator is bounded)."""
    rng = np.random.default_rng([43, seed])
    B, T, D = 2, 64, 6
    r = rng.uniform(-1, 1, (B, T, D)).astype(np.float32)
    s = (rng.uniform(-1, 1, (B, T, D)) - 0.5).astype(np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    out, _ = scan(r, s, x0)
    for b in range(B):
        for d in range(D):
            pool = np.concatenate([[x0[b, d]], r[b, :, d], s[b, :, d]]).astype(np.float32)
            bits = set(pool.view(np.uint32).tolist())
            col = out[b, :, d].astype(np.float32)
            if not set(col.view(np.uint32).tolist()) <= bits:
                return False
            if col.min() < pool.min() or col.max() > pool.max():
                return False
    return True


def minmax_brute_ok(scan, seed=0) -> bool:
    """Sequential scan against a per-element Python loop of the definition on a
    tiny case, fp32, bit for bit (brute force on tiny inputs)."""
    rng = np.random.default_rng([44, seed])
    B, T, D = 1, 9, 3
    r = rng.uniform(-1, 1, (B, T, D)).astype(np.float32)
    s = (rng.uniform(-1, 1, (B, T, D)) - 0.5).astype(np.float32)
    x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
    out, _ = scan(r, s, x0)
    for d in range(D):
        x = float(x0[0, d])
        for t in range(T):
            rt, st = float(r[0, t, d]), float(s[0, t, d])
            m = rt if rt < x else x
            x = st if st > m else m
            if np.float32(x) != out[0, t, d]:
                return False
    return True


def _all_groupings(items, combine):
    """Every full parenthesisation of a left-to-right combine of ``items``."""
    if len(items) == 1:
        yield items[0]
        return
    for cut in range(1, len(items)):
        for left in _all_groupings(items[:cut], combine):
            for right in _all_groupings(items[cut:], combine):
                yield combine(left, right)


def minmax_groupings_ok(compose, apply, seed=0, T=6, trials=20) -> bool:
    """Every parenthesisation of the composed clamp maps, applied to x_0, gives
    the sequential x_T bit for bit (including steps with s > r)."""
    rng = np.random.default_rng([45, seed])
    for _ in range(trials):
        r = rng.uniform(-1, 1, T).astype(np.float32)
        s = (rng.uniform(-1, 1, T) - 0.5).astype(np.float32)
        x0 = np.float32(rng.uniform(-1, 1))
        x = x0
        for t in range(T):
            x = np.float32(max(min(r[t], x), s[t]))
        maps = [(np.float32(r[t]), np.float32(s[t])) for t in range(T)]
        for m in _all_groupings(maps, compose):
            if np.float32(apply(m, x0)).view(np.uint32) != np.float32(x).view(np.uint32):
                return False
    return True


def logpair_groupings_err(pair_combine, seed=0, T=6) -> float:
    """Every parenthesisation of the log-pair composition gives the same
    (L, V) as the sequential left fold (up to rounding)."""
    rng = np.random.default_rng([46, seed])
    la = -rng.uniform(0.01, 3.0, T)
    lb = rng.normal(0.0, 2.0, T)
    pairs = [(la[t], lb[t]) for t in range(T)]
    seq = pairs[0]
    for pr in pairs[1:]:
        seq = pair_combine(seq, pr)
    worst = 0.0
    for m in _all_groupings(pairs, pair_combine):
        worst = max(worst, abs(m[0] - seq[0]), abs(m[1] - seq[1]))
    # And the pair means the affine map h -> e^L h + e^V.
    h = 0.37
    hseq = h
    for t in range(T):
        hseq = np.exp(la[t]) * hseq + np.exp(lb[t])
    worst = max(worst, abs(np.exp(seq[0]) * h + np.exp(seq[1]) - hseq) / abs(hseq))
    return worst


def all_groupings_count(n: int) -> int:
    """Catalan(n-1): used to check the enumeration is exhaustive."""
    return sum(1 for _ in _all_groupings(list(range(n)), lambda a, b: (a, b)))

