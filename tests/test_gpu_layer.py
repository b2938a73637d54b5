"""GPU parity of the full minGRU layer (projections on the matrix cores, the
scan, the output projection) and of the single-token step, against the fp64
oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import synth
from oracle import metrics, mingru
from tests.gpu_util import TOL_F32, dev, host64, say

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _layer_inputs(workload):
    cfg = synth.CONFIGS[workload]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    x = synth.normal_bt(workload, "x", B, T, D)
    W_in = synth.normal_mat(workload, "W_in", D, 2 * D, cfg["w_std"])
    W_out = synth.normal_mat(workload, "W_out", D, D, cfg["w_std"])
    return x, W_in, W_out


def _check_layer(x, W_in, W_out, h0=None, tol=TOL_F32):
    y, last = sr.mingru_forward(dev(x), dev(W_in), W_out=None if W_out is None else dev(W_out),
                                h0=None if h0 is None else dev(h0), return_last=True)
    y_ref, h_ref, last_ref = mingru.layer(x, W_in, W_out, h0)
    k, p = mingru.layer_kp(x, W_in)
    carry, inp = mingru.scan_terms(k, p, h0)
    if W_out is None:
        err = metrics.h_rel_err(host64(y), h_ref, carry, inp)
    else:
        err = metrics.y_rel_err(host64(y), y_ref, h_ref, W_out)
    err_last = metrics.h_rel_err(host64(last)[:, None], h_ref[:, -1:], carry[:, -1:], inp[:, -1:])
    say("layer err", err, "last err", err_last)
    assert err < tol and err_last < tol, (err, err_last)
    return y


@pytest.mark.parametrize("workload", [synth.LAYER_TINY, synth.LAYER])
def test_layer_workloads_match_oracle(workload):
    say(f"layer workload {workload}")
    x, W_in, W_out = _layer_inputs(workload)
    y = _check_layer(x, W_in, W_out)
    assert tuple(y.shape) == x.shape  # output has the input's shape


@pytest.mark.parametrize("B,T,D_in,D_h,D_out,with_out,with_h0", [
    (3, 77, 50, 37, 29, True, True),      # nothing divides anything
    (2, 300, 128, 96, 96, False, False),  # no output projection
    (1, 5, 3, 2, 7, True, False),          # tiny K
    (2, 130, 260, 130, 64, True, True),    # several M, N, K tiles with tails
])
def test_layer_ragged_shapes(B, T, D_in, D_h, D_out, with_out, with_h0):
    say(f"layer ragged {B} {T} {D_in} {D_h} {D_out}")
    rng = np.random.default_rng([700, B, T, D_in])
    x = rng.standard_normal((B, T, D_in)).astype(np.float32)
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / np.sqrt(D_in)).astype(np.float32)
    W_out = (rng.standard_normal((D_h, D_out)) / np.sqrt(D_h)).astype(np.float32) if with_out else None
    h0 = rng.uniform(0, 1, (B, D_h)).astype(np.float32) if with_h0 else None
    _check_layer(x, W_in, W_out, h0)


def test_step_loop_matches_oracle_and_parallel_mode():
    """Sequential mode of the B=2, T=1024, D=512 layer: 1024 token steps from a zero state, each
    checked against the oracle's step, and the final state against the
    parallel forward (the pages' parallel-vs-sequential comparison)."""
    say("step loop B=2 T=1024 D=512")
    x, W_in, W_out = _layer_inputs(synth.LAYER)
    B, T, D = x.shape
    xd, Wi, Wo = dev(x), dev(W_in), dev(W_out)
    y_par, h_par = sr.mingru_forward(xd, Wi, W_out=Wo, return_last=True)
    h = None
    ys = []
    for t in range(T):
        y_t, h = sr.mingru_step(xd[:, t].contiguous(), Wi, Wo, h_prev=h)
        ys.append(y_t)
    y_seq = torch.stack(ys, dim=1)
    y_ref, h_all, last_ref = mingru.layer(x, W_in, W_out)
    err = metrics.y_rel_err(host64(y_seq), y_ref, h_all, W_out)
    say("step err", err)
    assert err < TOL_F32
    # Parallel mode and sequential mode agree with each other.
    assert float((y_seq - y_par).abs().max()) < 1e-4 * float(y_par.abs().max())
    assert float((h - h_par).abs().max()) < 1e-5


def test_step_in_place_and_without_output_projection():
    rng = np.random.default_rng(701)
    B, D_in, D_h = 5, 33, 70
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / np.sqrt(D_in)).astype(np.float32)
    xs = rng.standard_normal((6, B, D_in)).astype(np.float32)
    Wi = dev(W_in)
    h = torch.zeros((B, D_h), device="cuda")
    h_ref = np.zeros((B, D_h))
    for t in range(6):
        y_t, h2 = sr.mingru_step(dev(xs[t]), Wi, None, h_prev=h, h_next=h)  # in place
        assert h2.data_ptr() == h.data_ptr() and y_t.data_ptr() == h.data_ptr()
        _, h_ref = mingru.step(xs[t], W_in, None, h_ref)
        assert np.max(np.abs(host64(h) - h_ref) / np.abs(h_ref)) < 1e-5


def test_layer_object_api():
    torch.manual_seed(0)
    layer = sr.MinGRU(64)
    x = torch.randn(2, 40, 64, device="cuda")
    y = layer(x)
    assert y.shape == x.shape
    # Token by token with the carried state matches the parallel call.
    prev = None
    outs = []
    for x_t in x.unbind(dim=1):
        y_t, prev = layer(x_t, prev_hidden=prev, return_next_prev_hidden=True)
        outs.append(y_t)
    y_seq = torch.stack(outs, dim=1)
    assert float((y_seq - y).abs().max()) < 1e-4 * float(y.abs().max())
    # The per-token step returns the new hidden state (the base step of the
    # tutorial: a (4, 32) token and hidden size 64 give a (4, 64) state).
    small = sr.MinGRU(32, expansion=2.0, W_out=False)
    y_t, h_t = small(torch.randn(4, 32, device="cuda"), None, return_next_prev_hidden=True)
    assert tuple(h_t.shape) == (4, 64) and tuple(y_t.shape) == (4, 64)


def test_decode_b256_d2048():
    """Decode workload: B=256 streams, D=2048; a parallel prefill of 512 steps, then
    4096 single-token steps carrying h.  Every one of the 256 rows is checked
    against the fp64 oracle after steps 1, 2, 8 (where the prefill's carry is
    still visible) and at the end; the oracle runs the whole 4608-step
    sequence, its projections (fp64 BLAS) streamed by blocks of 512 steps.
    The final state must also match the parallel forward over the
    concatenated sequence."""
    from oracle import mingru as orc
    cfg = synth.CONFIGS[synth.STEP]
    B, D, Tp, S = cfg["B"], cfg["D"], cfg["T_prefill"], cfg["steps"]
    say("decode B=256 D=2048")
    W_in = synth.device_normal(synth.STEP, "W_in", (D, 2 * D), 0.0, cfg["w_std"])
    W_out = synth.device_normal(synth.STEP, "W_out", (D, D), 0.0, cfg["w_std"])
    x = synth.device_normal(synth.STEP, "x", (B, Tp + S, D))
    _, h = sr.mingru_forward(x[:, :Tp], W_in, W_out=W_out, return_last=True)
    checks = (1, 2, 8)
    snaps = {}
    for t in range(S):
        y_t, h = sr.mingru_step(x[:, Tp + t].contiguous(), W_in, W_out, h_prev=h)
        if t + 1 in checks:
            snaps[Tp + t + 1] = h.double().cpu().numpy()
    snaps[Tp + S] = h.double().cpu().numpy()
    y_full, h_full = sr.mingru_forward(x, W_in, W_out=W_out, return_last=True)
    rel = float((h - h_full).abs().max() / h_full.abs().max())
    say("decode vs parallel", rel)
    assert rel < 1e-4
    # The oracle on all rows: h_t for t = 1 .. 4608 from the zero state, one
    # block of 512 steps at a time (the block's projection, then the scan
    # from the state the previous block left).
    Wi = W_in.double().cpu().numpy()
    ref = {}
    state = None
    blk = synth.T_BLOCK
    for t0 in range(0, Tp + S, blk):
        xb = x[:, t0:t0 + blk].double().cpu().numpy()
        k, p = orc.layer_kp(xb, Wi)
        hb = orc.scan(k, p, state)
        for step in snaps:
            if t0 < step <= t0 + blk:
                ref[step] = hb[:, step - 1 - t0].copy()
        state = hb[:, -1].copy()
        say(f"decode oracle: steps {t0 + 1}..{t0 + blk} done")
    for step, got in snaps.items():
        e = float(np.max(np.abs(got - ref[step]) / np.abs(ref[step])))
        say("decode step", step, "all rows, err", e)
        assert e < TOL_F32, (step, e)


@pytest.mark.parametrize("B,T,D_h,D_out", [
    (4, 8192, 256, 1024),     # 128 x 8 tiles of 256 x 128: the large-product path
    (3, 5000, 200, 1100),     # ragged rows, columns and K
])
def test_large_output_projection(B, T, D_h, D_out):
    """y = h W_out on a product large enough for the 256-row tiles, from a
    scan-only forward (k, p given)."""
    say(f"large W_out B={B} T={T} D_h={D_h} D_out={D_out}")
    rng = np.random.default_rng([1400, B, T])
    k = rng.normal(-1.0, 1.0, (B, T, D_h)).astype(np.float32)
    p = rng.standard_normal((B, T, D_h)).astype(np.float32)
    W_out = (rng.standard_normal((D_h, D_out)) / D_h ** 0.5).astype(np.float32)
    y = sr.mingru_forward(k=dev(k), p=dev(p), W_out=dev(W_out))
    h_ref = mingru.scan(k, p)
    y_ref = mingru.project(h_ref, W_out)
    err = metrics.y_rel_err(y.double().cpu().numpy(), y_ref, h_ref, W_out)
    say("error", err)
    assert err < TOL_F32


@pytest.mark.parametrize("B", [1, 5, 16, 17, 40])
def test_step_batch_sizes(B):
    """The step's products run on FMAs up to 16 streams and on the matrix
    cores above; both against the fp64 oracle, three steps carried."""
    say(f"step B={B}")
    rng = np.random.default_rng([1500, B])
    D_in, D_h, D_out = 96, 160, 80
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / D_in ** 0.5).astype(np.float32)
    W_out = (rng.standard_normal((D_h, D_out)) / D_h ** 0.5).astype(np.float32)
    h = dev(rng.standard_normal((B, D_h)).astype(np.float32))
    h_ref = host64(h)
    for t in range(3):
        x_t = rng.standard_normal((B, D_in)).astype(np.float32)
        y_t, h = sr.mingru_step(dev(x_t), dev(W_in), dev(W_out), h_prev=h)
        y_ref, h_ref = mingru.step(x_t, W_in, W_out, h_ref)
        assert metrics.max_abs_rel(host64(h), h_ref) < TOL_F32
        assert metrics.y_rel_err(host64(y_t), y_ref, h_ref, W_out) < TOL_F32
        h_ref = host64(h)


@pytest.mark.parametrize("B,D_in,D_h,decayed,path", [
    (5, 40, 96, False, "FMA path (<= 16 rows)"),
    (100, 72, 130, False, "narrow 32-row tiles, ragged"),
    (256, 256, 2048, False, "narrow 64-row tiles, full"),
    (256, 256, 2048, True, "narrow 64-row tiles, full, decayed"),
    (700, 1024, 256, False, "narrow tiles above 512 rows (K <= 1024)"),
    (700, 2048, 256, False, "128-row tiles with K split over workgroups"),
    (700, 2048, 256, True, "128-row tiles with K split, decayed"),
])
def test_step_in_place_on_every_path(B, D_in, D_h, decayed, path):
    """h_next may be h_prev: every product path reads each carried state
    before the same workgroup (or the split-K reduction) overwrites it.  The
    in-place step equals the out-of-place one bit for bit, and the oracle."""
    say(f"in-place step B={B} D_in={D_in} D_h={D_h} decayed={decayed}: {path}")
    rng = np.random.default_rng([1710, B, D_h, int(decayed)])
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / np.sqrt(D_in)).astype(np.float32)
    x_t = rng.standard_normal((B, D_in)).astype(np.float32)
    h0 = rng.standard_normal((B, D_h)).astype(np.float32)
    lam = (10.0 ** rng.uniform(-3, 0, D_h)).astype(np.float32)
    dt = rng.exponential(1.0, B).astype(np.float32)
    Wi, xd = dev(W_in), dev(x_t)

    def step(h_prev, h_next):
        if decayed:
            return sr.mingru_step_decayed(xd, Wi, None, h_prev=h_prev, h_next=h_next,
                                          decay_rate=dev(lam), delta_t=dev(dt))
        return sr.mingru_step(xd, Wi, None, h_prev=h_prev, h_next=h_next)

    _, apart = step(dev(h0), None)
    h = dev(h0)
    _, same = step(h, h)
    assert same.data_ptr() == h.data_ptr()
    assert torch.equal(h, apart)
    if decayed:
        from oracle import decay
        _, h_ref = decay.step(x_t, W_in, lam, dt, None, h0)
    else:
        _, h_ref = mingru.step(x_t, W_in, None, h0)
    assert metrics.max_abs_rel(host64(h), h_ref) < TOL_F32
