"""The oracle run over channel slices in worker processes gives exactly what
one process gives (every channel is its own recurrence): the same max error,
and every element counted once."""

import numpy as np

from oracle import metrics, mingru, parallel


def _inputs(seed, B=2, T=700, D=150):
    rng = np.random.default_rng(seed)
    k = rng.normal(-3.0, 1.5, (B, T, D)).astype(np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    return k, p, h0


def test_parallel_error_equals_serial_error():
    k, p, h0 = _inputs(1)
    ref = mingru.scan(k, p, h0)
    rng = np.random.default_rng(2)
    got = (ref * (1 + 1e-6 * rng.standard_normal(ref.shape))).astype(np.float32)
    got[1, 333, 77] *= 1.001  # one element far off: the max must find it
    carry, inp = mingru.scan_terms(k, p, h0)
    serial = metrics.h_rel_err(got, ref, carry, inp)
    assert serial > 1e-4
    assert parallel.mingru_scan_error(k, p, h0, got, workers=3, width=64) == serial
    assert parallel.mingru_scan_error(k, p, h0, got, workers=1, width=40) == serial


def test_slices_cover_every_channel_once():
    sl = parallel.channel_slices(3, 150, 64)
    seen = np.zeros((3, 150), int)
    for b, d0, d1 in sl:
        seen[b, d0:d1] += 1
    assert np.all(seen == 1)
    k, p, h0 = _inputs(3, B=3, T=50)
    res = parallel.mingru_scan_timed(k, p, h0, workers=2, width=64)
    assert res["elements"] == k.size and res["workers"] == 2
