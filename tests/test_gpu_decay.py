"""GPU parity of the time-decayed minGRU scan and step against the fp64 oracle."""

import warnings

import numpy as np
import pytest
import torch

import synth
from oracle import decay, metrics
from tests.gpu_util import TOL_F32, dev, host64, say
from tests import pins_decay

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _case(B, T, D, seed, huge=False):
    rng = np.random.default_rng([1200, seed])
    k = rng.normal(-1.0, 1.5, (B, T, D)).astype(np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    lam = (10.0 ** rng.uniform(-3, 0, D)).astype(np.float32)
    dt = rng.exponential(1.0, (B, T)).astype(np.float32)
    dt[rng.random((B, T)) < 0.05] = 0.0
    if huge:
        dt[rng.random((B, T)) < 0.01] = 1e6
    return k, p, h0, lam, dt


def _err(h, k, p, lam, dt, h0, log1p):
    ref = decay.scan(k, p, lam, dt, h0, log1p)
    carry, inp = decay.scan_terms(k, p, lam, dt, h0, log1p)
    return metrics.h_rel_err(host64(h), ref, carry, inp)


@pytest.mark.parametrize("B,T,D,with_h0,log1p,huge", [
    (2, 64, 16, False, False, False),
    (3, 1000, 200, True, False, True),
    (2, 5000, 384, True, True, True),
    (1, 1, 8, True, False, False),
    (4, 333, 7, False, True, False),
    (1, 7000, 130, True, False, True),
])
def test_decayed_scan_f32(B, T, D, with_h0, log1p, huge):
    say(f"decay f32 B={B} T={T} D={D} h0={with_h0} log1p={log1p} huge={huge}")
    k, p, h0, lam, dt = _case(B, T, D, seed=B * 7 + T + D, huge=huge)
    h0 = h0 if with_h0 else None
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    h, last = sr.mingru_forward_decayed(k=dev(k), p=dev(p), h0=None if h0 is None else dev(h0),
                                        decay_rate=dev(lam), delta_t=dev(dt), log1p_delta=log1p,
                                        saturated=sat, return_last=True)
    err = _err(h, k, p, lam, dt, h0, log1p)
    say("error", err)
    assert err < TOL_F32
    assert torch.equal(last, h[:, -1])
    assert int(sat.item()) == int(decay.saturated(lam, dt, log1p))


def test_decayed_scan_bf16_long_memory_reduced():
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = 2, 4096, 1024
    say("decay bf16 long-memory B=2 T=4096 D=1024")
    kb = synth.bf16_round(synth.normal_bt(synth.SCAN, "k", B, T, D, cfg["k_mean"], cfg["k_std"])).cuda()
    pb = synth.bf16_round(synth.normal_bt(synth.SCAN, "p", B, T, D, cfg["p_mean"], cfg["p_std"])).cuda()
    h0 = synth.normal_vec(synth.SCAN, "h0", B, D)
    lam = synth.decay_rates(synth.SCAN, D)
    dt = synth.gaps(synth.SCAN, B, T)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    h = sr.mingru_forward_decayed(k=kb, p=pb, h0=dev(h0), decay_rate=dev(lam), delta_t=dev(dt),
                                  saturated=sat)
    err = _err(h, kb.double().cpu().numpy(), pb.double().cpu().numpy(), lam, dt, h0, False)
    say("error", err)
    assert err < TOL_F32
    assert int(sat.item()) == int(decay.saturated(lam, dt)) == 1


def test_zero_gaps_equal_undecayed_bitwise():
    B, T, D = 2, 3000, 256
    k, p, h0, lam, _ = _case(B, T, D, seed=1201)
    kd, pd, h0d = dev(k), dev(p), dev(h0)
    plain = sr.mingru_forward(k=kd, p=pd, h0=h0d)
    dec = sr.mingru_forward_decayed(k=kd, p=pd, h0=h0d, decay_rate=dev(lam),
                                    delta_t=torch.zeros((B, T), device="cuda"))
    assert torch.equal(plain, dec)
    dec0 = sr.mingru_forward_decayed(k=kd, p=pd, h0=h0d, decay_rate=torch.zeros(D, device="cuda"),
                                     delta_t=dev(np.full((B, T), 3.0, np.float32)))
    assert torch.equal(plain, dec0)


def test_saturating_gap_restarts_the_state():
    """A gap far past the clamp wipes the carried state: from that token on,
    h equals a fresh scan of the remaining tokens (within rounding, as the
    tiles fall differently), and the flag is set; with log1p_delta the same
    gaps do not saturate."""
    B, T, D = 2, 9000, 192
    k, p, h0, lam, dt = _case(B, T, D, seed=1202)
    lam = np.maximum(lam, np.float32(0.05))
    tstar = 4321
    dt[:, tstar] = 1e7
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    kd, pd, lamd = dev(k), dev(p), dev(lam)
    h = sr.mingru_forward_decayed(k=kd, p=pd, h0=dev(h0), decay_rate=lamd, delta_t=dev(dt),
                                  saturated=sat)
    assert int(sat.item()) == 1
    dt_fresh = dt[:, tstar:].copy()
    dt_fresh[:, 0] = 0.0
    fresh = sr.mingru_forward_decayed(k=kd[:, tstar:].contiguous(), p=pd[:, tstar:].contiguous(),
                                      decay_rate=lamd, delta_t=dev(dt_fresh))
    ref = decay.scan(k[:, tstar:], p[:, tstar:], lam, dt_fresh)
    assert metrics.max_abs_rel(host64(h[:, tstar:]), ref) < 1e-5
    assert metrics.max_abs_rel(host64(fresh), ref) < 1e-5
    sat.zero_()
    sr.mingru_forward_decayed(k=kd, p=pd, h0=dev(h0), decay_rate=lamd, delta_t=dev(dt),
                              log1p_delta=True, saturated=sat)
    assert int(sat.item()) == 0


def test_page_example_through_the_layer():
    """The tutorial's Step 5 run, on the minGRU layer: the same token six
    times, gaps [0, 1, 1, 20000, 1, 1] against all-zero gaps, the state read
    after each prefix.  The gapped state after events 3, 4, 5 repeats events
    0, 1, 2 bit for bit; control equals the undecayed layer; one warning
    over the whole trajectory, none with log1p_delta."""
    D = 8
    g = torch.Generator().manual_seed(0)
    rate = torch.rand(D, generator=g) * 1.4 + 0.6        # rate * 20000 > 1e4 everywhere
    layer = sr.MinGRU(D, decay_rate=rate, generator=g)
    x = torch.randn(1, 1, D, generator=g).expand(1, 6, D).contiguous().cuda()
    gapped = torch.tensor([pins_decay.PAGE_GAPS]).cuda()
    control = torch.zeros_like(gapped)

    def trajectory(lyr, delta_t):
        states = []
        with warnings.catch_warnings(record=True) as caught:
            warnings.simplefilter("always")
            for t in range(1, 7):
                _, h = lyr(x[:, :t], delta_t=delta_t[:, :t], return_next_prev_hidden=True)
                states.append(h.clone())
        return torch.stack(states, 1)[0], list(caught)

    hg, wg = trajectory(layer, gapped)
    ctl = sr.MinGRU(D, W_in=layer.W_in, W_out=layer.W_out, decay_rate=rate)
    hc, wc = trajectory(ctl, control)
    assert len(wg) == 1 and issubclass(wg[0].category, UserWarning) and not wc
    assert torch.equal(hg[3:6], hg[0:3])
    assert torch.equal(hg[0], hc[0])
    _, plain = sr.MinGRU(D, W_in=layer.W_in, W_out=layer.W_out)(x, return_next_prev_hidden=True)
    assert torch.equal(hc[5], plain[0])
    ng, nc = hg.norm(dim=1), hc.norm(dim=1)
    assert bool((nc[1:] >= nc[:-1]).all()) and bool((ng[1:3] < nc[1:3]).all())
    soft = sr.MinGRU(D, W_in=layer.W_in, W_out=layer.W_out, decay_rate=rate, log1p_delta=True)
    _, ws = trajectory(soft, gapped)
    assert not ws


def test_decayed_step_loop_matches_oracle():
    """Token by token with W_in / W_out (the step kernel's epilogue applies
    the decay), against the oracle's step, carrying h between calls."""
    rng = np.random.default_rng(1203)
    B, T, D_in, D_h = 4, 40, 96, 160
    x = rng.standard_normal((B, T, D_in)).astype(np.float32)
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / D_in ** 0.5).astype(np.float32)
    W_out = (rng.standard_normal((D_h, D_h)) / D_h ** 0.5).astype(np.float32)
    lam = (10.0 ** rng.uniform(-2, 0, D_h)).astype(np.float32)
    dt = rng.exponential(1.0, (B, T)).astype(np.float32)
    dt[:, 17] = 1e6
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    Wi, Wo, lamd, dtd = dev(W_in), dev(W_out), dev(lam), dev(dt)
    h = None
    h_ref = None
    for t in range(T):
        y_t, h = sr.mingru_step_decayed(dev(x[:, t]), Wi, Wo, h, decay_rate=lamd,
                                        delta_t=dtd[:, t].contiguous(), log1p_delta=False,
                                        saturated=sat)
        y_ref, h_ref = decay.step(x[:, t], W_in, lam, dt[:, t], W_out, h_ref)
        assert metrics.max_abs_rel(host64(h), h_ref) < 1e-4, t
        assert metrics.y_rel_err(host64(y_t), y_ref, h_ref, W_out) < 1e-4, t
        h_ref = host64(h)   # carry the GPU state, so each step is checked on its own
    assert int(sat.item()) == 1
    # The whole-sequence call on the same inputs agrees with the oracle too.
    y, last = sr.mingru_forward_decayed(dev(x), Wi, W_out=Wo, decay_rate=lamd, delta_t=dtd,
                                        return_last=True)
    y_ref, hs_ref, _ = decay.layer(x, W_in, lam, dt, W_out)
    assert metrics.y_rel_err(host64(y), y_ref, hs_ref, W_out) < 1e-4


def test_full_size_b8_t65536_d1024_decayed_every_element():
    """The decayed scan at the bench workload's full size, with gaps that
    saturate: every output against the fp64 oracle (worker processes)."""
    from tests import fullsize
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    say("decay full size B=8 T=65536 D=1024, every element")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    lam = synth.decay_rates(synth.SCAN, D)
    dt = synth.gaps(synth.SCAN, B, T)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    h = sr.mingru_forward_decayed(k=kb, p=pb, h0=h0, decay_rate=dev(lam), delta_t=dev(dt),
                                  saturated=sat, workspace=ws)
    assert sr.workspace_status(ws) == 0
    assert int(sat.item()) == 1
    H = fullsize.host32
    arrays = dict(k=H(kb), p=H(pb), h0=H(h0), got=H(h), lam=lam, dt=dt,
                  log1p=np.zeros(1, np.int32))
    del kb, pb, h
    torch.cuda.empty_cache()
    say("oracle on every channel")
    err = max(fullsize.all_channels(fullsize.decayed_slice_error, arrays, B, D))
    say("decayed full size error (every element)", err)
    assert err < TOL_F32


def test_decayed_step_over_many_streams():
    """1024 streams with D_in = 2048: the input product splits K across
    workgroups, and the reduction kernel applies the decayed update."""
    B, D_in, D_h = 1024, 2048, 512
    say("decayed step B=1024")
    assert sr.raw_library().mingru_step_workspace_size(B, D_in, D_h, D_h) > 0
    rng = np.random.default_rng(1204)
    x_t = rng.standard_normal((B, D_in)).astype(np.float32)
    W_in = (rng.standard_normal((D_in, 2 * D_h)) / D_in ** 0.5).astype(np.float32)
    lam = (10.0 ** rng.uniform(-3, 0, D_h)).astype(np.float32)
    dt = rng.exponential(1.0, B).astype(np.float32)
    dt[::97] = 1e6
    h0 = rng.standard_normal((B, D_h)).astype(np.float32)
    for log1p in (False, True):
        sat = torch.zeros(1, dtype=torch.int32, device="cuda")
        _, h = sr.mingru_step_decayed(dev(x_t), dev(W_in), h_prev=dev(h0), decay_rate=dev(lam),
                                      delta_t=dev(dt), log1p_delta=log1p, saturated=sat)
        _, h_ref = decay.step(x_t, W_in, lam, dt, None, h0, log1p)
        err = metrics.max_abs_rel(host64(h), h_ref)
        say("log1p", log1p, "error", err)
        assert err < TOL_F32
        assert int(sat.item()) == int(decay.saturated(lam, dt, log1p))


def test_long_memory_with_small_decays_closed_form():
    """Constant gates that keep almost all of the state (z from 6e-6 to 2.5e-3)
    and constant small decays (x = rate * gap from 1e-6 to 1e-4), over 65536
    steps crossing hundreds of tiles: each step's coefficient A = sigma(-k)
    e^{-x} lies within 1e-3 of 1, and the result has the geometric closed
    form h_t = A^t h0 + b (1 - A^t) / (1 - A), b = sigma(k) g(p), evaluated
    in fp64 from the same fp32 inputs.  The complement 1 - A must stay
    accurate through every composition (a cancelling 1 - e^{-x} would be off
    by ~1e-3 relative here)."""
    B, T, D = 2, 65536, 256
    say(f"decayed long memory closed form B={B} T={T} D={D}")
    rng = np.random.default_rng(1207)
    k_ch = rng.uniform(-12.0, -6.0, (B, D)).astype(np.float32)
    p_ch = rng.uniform(0.2, 2.0, (B, D)).astype(np.float32)
    lam = (10.0 ** rng.uniform(-6.0, -4.0, D)).astype(np.float32)
    gap = np.float32(1.0)
    h0 = rng.uniform(0.5, 2.0, (B, D)).astype(np.float32)
    k = np.broadcast_to(k_ch[:, None, :], (B, T, D))
    p = np.broadcast_to(p_ch[:, None, :], (B, T, D))
    dt = np.full((B, T), gap, np.float32)
    h = sr.mingru_forward_decayed(k=dev(k), p=dev(p), h0=dev(h0), decay_rate=dev(lam),
                                  delta_t=dev(dt))
    torch.cuda.synchronize()
    # closed form in fp64 (A, b as functions of the fp32 inputs)
    k64, p64, x = k_ch.astype(np.float64), p_ch.astype(np.float64), lam.astype(np.float64) * 1.0
    z = 1.0 / (1.0 + np.exp(-k64))
    a = 1.0 / (1.0 + np.exp(k64))
    log_A = -np.log1p(np.exp(k64)) - x[None, :]          # log(sigma(-k)) - x
    one_minus_A = -np.expm1(log_A)
    bstep = z * (p64 + 0.5)
    ts = np.array([1, 2, 100, 1000, 10000, 30000, 65536])
    got = host64(h)[:, ts - 1, :]
    At = np.exp(ts[None, :, None] * log_A[:, None, :])
    carry = At * h0.astype(np.float64)[:, None, :]
    inp = bstep[:, None, :] * (-np.expm1(ts[None, :, None] * log_A[:, None, :])) / one_minus_A[:, None, :]
    ref = carry + inp
    err = float(np.max(np.abs(got - ref) / (np.abs(carry) + np.abs(inp))))
    say("max conditioned error", err, "A^T range", float(At[..., -1].min()), float(At[..., -1].max()))
    assert err < TOL_F32
