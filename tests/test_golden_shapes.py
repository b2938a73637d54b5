"""The pages' printed shape contracts, checked on the oracle."""

import os

import numpy as np

from oracle import minmax, mingru

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "shapes.txt")


def _cases():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, inp, out, src = [c.strip() for c in line.split("|")]
                rows[name] = (inp, out, src)
    return rows


def test_fixture_lists_its_sources():
    rows = _cases()
    assert set(rows) == {"layer_parallel", "step_hidden", "minmax_state"}
    assert all(src for _, _, src in rows.values())


def test_parallel_layer_keeps_the_input_shape():
    x = np.zeros((2, 1024, 512))
    W_in = np.zeros((512, 1024))
    W_out = np.zeros((512, 512))
    y, h, last = mingru.layer(x, W_in, W_out)
    assert y.shape == (2, 1024, 512) and last.shape == (2, 512)


def test_step_maps_token_to_hidden():
    x_t = np.ones((4, 32))
    W_in = np.zeros((32, 128))
    y_t, h_t = mingru.step(x_t, W_in)
    assert h_t.shape == (4, 64) and y_t.shape == (4, 64)


def test_minmax_state_width():
    r = np.zeros((1, 3, 192), np.float32)
    out, last = minmax.scan(r, r, np.zeros((1, 192), np.float32))
    assert out.shape == (1, 3, 192) and last.shape == (1, 192)
