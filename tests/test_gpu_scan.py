"""GPU parity of the minGRU scan (scan-only calls of mingru_forward) against
the fp64 sequential oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import synth
from oracle import mingru, scalar
from tests.gpu_util import TOL_BF16, TOL_F32, dev, host64, say, scan_err

pytestmark = pytest.mark.gpu

sr = pytest.importorskip("scan_linear_rnn_amd")


def _inputs(B, T, D, seed, k_mean=0.0, k_std=1.5, with_h0=True):
    rng = np.random.default_rng([500, seed])
    k = (k_mean + k_std * rng.standard_normal((B, T, D))).astype(np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32) if with_h0 else None
    return k, p, h0


@pytest.mark.parametrize("B,T,D,with_h0", [
    (2, 64, 16, False),        # the tiny layer's scan shape
    (3, 1000, 200, True),      # ragged T and D, several tiles along T
    (2, 4096, 512, True),      # many tiles, look-back chains
    (1, 1, 8, True),           # one step
    (2, 2, 3, False),          # D with no vector width
    (1, 333, 130, True),       # D = 2 * 65: ragged lanes
    (4, 2500, 64, False),
    # At least 32 chains (batch rows x 128-channel tiles): two channels per
    # lane; the shapes above take one channel per lane.
    (32, 1000, 200, True),     # ragged T and D
    (16, 700, 1000, True),     # D = 1000: the last 128-channel tile part full
])
def test_scan_f32_matches_oracle(B, T, D, with_h0):
    say(f"scan f32 B={B} T={T} D={D} h0={with_h0}")
    k, p, h0 = _inputs(B, T, D, seed=B * 7 + T + D, with_h0=with_h0)
    y, last = sr.mingru_forward(k=dev(k), p=dev(p), h0=None if h0 is None else dev(h0),
                                return_last=True)
    err = scan_err(host64(y), k, p, h0)
    assert err < TOL_F32, err
    assert np.array_equal(host64(last), host64(y)[:, -1, :])


@pytest.mark.parametrize("B", [2, 4])  # 16 chains (one channel per lane), 32 (two)
def test_scan_bf16_long_memory_statistics(B):
    T, D = 4096, 1024
    say(f"scan bf16 long-memory B={B} T={T} D={D}")
    cfg = synth.CONFIGS[synth.SCAN]
    k32 = synth.normal_bt(synth.SCAN, "k", B, T, D, cfg["k_mean"], cfg["k_std"])
    p32 = synth.normal_bt(synth.SCAN, "p", B, T, D, cfg["p_mean"], cfg["p_std"])
    h0 = synth.normal_vec(synth.SCAN, "h0", B, D)
    kb, pb = synth.bf16_round(k32), synth.bf16_round(p32)
    y = sr.mingru_forward(k=kb.cuda(), p=pb.cuda(), h0=dev(h0))
    # The oracle reads the same bf16 values.
    err = scan_err(host64(y), kb.double().numpy(), pb.double().numpy(), h0)
    say("bf16 err", err)
    assert err < TOL_BF16
    assert err < 1e-5  # the arithmetic itself is fp32: regressions show long before 2e-2


@pytest.mark.parametrize("B", [2, 32])  # one / two channels per lane
def test_scan_kp_halves_of_one_buffer(B):
    T, D = 700, 96
    say(f"scan ld_kp != D_h, B={B}")
    rng = np.random.default_rng(77)
    kp = rng.standard_normal((B, T, 2 * D)).astype(np.float32)
    t = dev(kp)
    y = sr.mingru_forward(k=t[..., :D], p=t[..., D:])
    assert scan_err(host64(y), kp[..., :D], kp[..., D:], None) < TOL_F32


def test_long_memory_closed_forms_cross_many_tiles():
    # k = -30: sigma(-30) = 9.4e-14, so h_t = h_0 across every tile.
    B, T, D = 2, 20000, 256
    say("long memory k=-30")
    rng = np.random.default_rng(78)
    k = np.full((B, T, D), -30.0, np.float32)
    p = rng.standard_normal((B, T, D)).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    y = host64(sr.mingru_forward(k=dev(k), p=dev(p), h0=dev(h0)))
    assert np.max(np.abs(y - h0[:, None, :])) < 1e-6
    # k_1 = +30 then -30: the first step writes g(p_1), which is then held.
    k[:, 0, :] = 30.0
    y = host64(sr.mingru_forward(k=dev(k), p=dev(p), h0=dev(h0)))
    g1 = scalar.g(p[:, 0, :].astype(np.float64))
    assert np.max(np.abs(y - g1[:, None, :]) / g1[:, None, :]) < 1e-5


def test_z_one_gives_candidate():
    B, T, D = 2, 3000, 128
    rng = np.random.default_rng(79)
    k = np.full((B, T, D), 30.0, np.float32)
    p = (3 * rng.standard_normal((B, T, D))).astype(np.float32)
    y = host64(sr.mingru_forward(k=dev(k), p=dev(p), h0=dev(np.ones((B, D), np.float32))))
    g = scalar.g(p.astype(np.float64))
    assert np.max(np.abs(y - g) / g) < 1e-5


def test_repeated_calls_are_bitwise_identical():
    B, T, D = 4, 8192, 512
    k, p, h0 = _inputs(B, T, D, seed=80, k_mean=-4.0, k_std=1.0)
    kd, pd, hd = dev(k), dev(p), dev(h0)
    ref = sr.mingru_forward(k=kd, p=pd, h0=hd)
    for _ in range(3):
        out = sr.mingru_forward(k=kd, p=pd, h0=hd)
        assert torch.equal(out, ref)


def test_carried_state_concatenation():
    B, T, D = 2, 3000, 256
    k, p, h0 = _inputs(B, T, D, seed=81)
    kd, pd, hd = dev(k), dev(p), dev(h0)
    y, last = sr.mingru_forward(k=kd, p=pd, h0=hd, return_last=True)
    T1 = 1234
    y1, l1 = sr.mingru_forward(k=kd[:, :T1], p=pd[:, :T1], h0=hd, return_last=True)
    y2, l2 = sr.mingru_forward(k=kd[:, T1:], p=pd[:, T1:], h0=l1, return_last=True)
    joined = host64(torch.cat([y1, y2], dim=1))
    assert scan_err(joined, k, p, h0) < TOL_F32
    assert np.max(np.abs(joined - host64(y))) < 1e-5


def test_empty_sequence_returns_carried_state():
    B, D = 3, 40
    h0 = dev(np.arange(B * D, dtype=np.float32).reshape(B, D))
    k = torch.zeros((B, 0, D), device="cuda")
    y, last = sr.mingru_forward(k=k, p=k, h0=h0, return_last=True)
    assert y.shape == (B, 0, D) and torch.equal(last, h0)
    y, last = sr.mingru_forward(k=k, p=k, return_last=True)
    assert torch.count_nonzero(last) == 0


def test_full_size_b8_t65536_d1024_every_element():
    """The bench workload at full size (B=8, T=65536, D=1024, bf16 inputs),
    launched exactly as the benchmark launches it: every one of the 2^29
    outputs and h_T against the fp64 oracle (run on every channel in worker
    processes)."""
    from oracle import parallel
    from tests import fullsize
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    say("full size B=8 T=65536 D=1024, every element")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    y, last = sr.mingru_forward(k=kb, p=pb, h0=h0, return_last=True, workspace=ws)
    assert sr.workspace_status(ws) == 0
    assert bool(torch.isfinite(y).all())
    assert torch.equal(last, y[:, -1])
    k, p, hh0, got = fullsize.host32(kb), fullsize.host32(pb), fullsize.host32(h0), fullsize.host32(y)
    del kb, pb, y
    torch.cuda.empty_cache()
    say("oracle on every channel")
    err = parallel.mingru_scan_error(k, p, hh0, got)
    say("full size error (every element)", err)
    assert err < TOL_BF16 and err < 1e-5


def test_caller_workspace_is_checked():
    """A workspace passed by the caller is used as given or rejected, never
    silently replaced."""
    k = torch.zeros((2, 300, 64), device="cuda")
    n = sr.raw_library().mingru_forward_workspace_size(2, 300, 0, 64, 64, 0, 0)
    good = torch.empty(n, dtype=torch.uint8, device="cuda")
    sr.mingru_forward(k=k, p=k, workspace=good)
    with pytest.raises(ValueError):
        sr.mingru_forward(k=k, p=k, workspace=good[: n - 1])
    with pytest.raises(TypeError):
        sr.mingru_forward(k=k, p=k, workspace=torch.empty(n, device="cuda"))
    with pytest.raises(ValueError):
        sr.minmax_scan(k, k, torch.zeros((2, 64), device="cuda"), workspace=good[:16])


def test_one_workspace_reused_across_shapes_and_ops():
    """One caller workspace serves a run of calls of different shapes, input
    types and operators (the scan's look-back words, the MinMax scan's, the
    backward's) in one stream: every call resets what it uses, so no earlier
    call's words leak into a later one."""
    from oracle import minmax
    lib = sr.raw_library()
    shapes = [(2, 4096, 512), (3, 1000, 200), (1, 7000, 64), (2, 4096, 512), (4, 300, 1030)]
    n = max(max(lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                lib.minmax_scan_workspace_size(B, T, D),
                lib.mingru_scan_backward_workspace_size(B, T, D)) for B, T, D in shapes)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for i, (B, T, D) in enumerate(shapes):
        say(f"reuse {i}: B={B} T={T} D={D}")
        k, p, h0 = _inputs(B, T, D, seed=900 + i)
        bf16 = i % 2 == 1
        kd = dev(k).to(torch.bfloat16) if bf16 else dev(k)
        pd = dev(p).to(torch.bfloat16) if bf16 else dev(p)
        h = sr.mingru_forward(k=kd, p=pd, h0=dev(h0), workspace=ws)
        kk, pp = (host64(kd), host64(pd)) if bf16 else (k, p)
        err = scan_err(host64(h), kk, pp, h0)
        assert err < (TOL_BF16 if bf16 else TOL_F32), (i, err)
        rng = np.random.default_rng([901, i])
        r = rng.uniform(-1, 1, (B, T, D)).astype(np.float32)
        s = rng.uniform(-1.5, 0.5, (B, T, D)).astype(np.float32)
        x0 = rng.uniform(-1, 1, (B, D)).astype(np.float32)
        x = sr.minmax_scan(dev(r), dev(s), dev(x0), workspace=ws)
        assert np.array_equal(host64(x), minmax.scan(r, s, x0)[0]), i
        # A backward call between forwards leaves its own words behind.
        sr.mingru_scan_backward(kd, pd, h, torch.ones_like(h), workspace=ws)


def _closed_form_check(B, T, D, kc, pc, h0, dtype):
    """Constant k and p per channel: h_t = a^t h_0 + b (1 - a^t) / (1 - a), a =
    sigma(-k), b = sigma(k) g(p) (a geometric series), at sampled steps of
    every channel, conditioned as the oracle's error measure.  1 - a is
    sigma(k) itself, so the series is evaluated without cancellation."""
    k = torch.from_numpy(kc).cuda()[None, None, :].expand(B, T, D).to(dtype).contiguous()
    p = torch.from_numpy(pc).cuda()[None, None, :].expand(B, T, D).to(dtype).contiguous()
    kc64 = k[0, 0].double().cpu().numpy()  # the values the kernel reads
    pc64 = p[0, 0].double().cpu().numpy()
    y = sr.mingru_forward(k=k, p=p, h0=dev(h0))
    del k, p
    rng = np.random.default_rng([81, T])
    ts = np.unique(np.concatenate([[1, 2, 143, 144, 145, 288, 289, 4096, T // 2, T - 1, T],
                                   rng.integers(1, T + 1, 48)]))
    got = host64(y[:, torch.from_numpy(ts - 1).to(y.device), :])
    a = scalar.sigmoid(-kc64)
    c = scalar.sigmoid(kc64)                                          # 1 - a
    b = c * scalar.g(pc64)
    # a^t = exp(-t softplus(k)) and 1 - a^t = -expm1(-t softplus(k)).
    lt = ts[:, None].astype(np.float64) * scalar.softplus(kc64)[None, :]
    at = np.exp(-lt)
    carry = at[None] * h0.astype(np.float64)[:, None, :]
    inp = (b * -np.expm1(-lt) / c)[None]
    ref = carry + inp
    err = np.max(np.abs(got - ref) / (np.abs(carry) + inp))
    return err


def test_long_memory_closed_form_across_thousands_of_tiles():
    """T = 2^20 + 5 in one chain per (batch row, channel tile): the state
    crosses ~3600 tiles through the look-back.  Memory lengths up to
    1/sigma(-12) ~ 1.6e5 steps (k in [-12, 2]), the regime where the
    retained fraction 1 - sigma(k) is far below an ulp of 1: the scan carries
    the complement of every composed coefficient, so the fixed point b/(1-a)
    is reached to a few ulps (a product of rounded coefficients would be off
    by ulp/(1-a), 1e-3 relative at k = -10).  D = 130: a ragged channel tile
    (one channel per lane, 288-step tiles)."""
    B, T, D = 2, (1 << 20) + 5, 130
    say(f"closed form B={B} T={T} D={D}")
    rng = np.random.default_rng(81)
    kc = np.concatenate([[-12.0, -11.0, -10.0, -9.0, -8.0, -6.0, -4.0, 2.0],
                         rng.uniform(-12.0, 2.0, D - 8)]).astype(np.float32)
    pc = rng.standard_normal(D).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    err = _closed_form_check(B, T, D, kc, pc, h0, torch.float32)
    say("closed-form error", err)
    assert err < TOL_F32


def test_long_memory_closed_form_two_channels_per_lane():
    """The same closed form on the other tile geometry (two channels per lane,
    144-step tiles, 64 chains) with bf16 gate logits, k in [-12, 2], over
    2^17 steps (~900 tiles per chain)."""
    B, T, D = 32, 1 << 17, 256
    say(f"closed form B={B} T={T} D={D} bf16")
    rng = np.random.default_rng(83)
    kc = np.concatenate([[-12.0, -10.0, -8.0, 2.0], rng.uniform(-12.0, 2.0, D - 4)]).astype(np.float32)
    pc = rng.standard_normal(D).astype(np.float32)
    h0 = rng.standard_normal((B, D)).astype(np.float32)
    err = _closed_form_check(B, T, D, kc, pc, h0, torch.bfloat16)
    say("closed-form error", err)
    assert err < TOL_F32


def test_two_streams_at_once():
    """Two scans in flight together on two streams (separate workspaces):
    their tiles interleave on the GPU; each result equals the same call made
    alone, bit for bit, and the oracle."""
    shapes = [(4, 8192, 512), (2, 20000, 256)]
    ins = [_inputs(B, T, D, seed=82 + i, k_mean=-4.0, k_std=1.0) for i, (B, T, D) in enumerate(shapes)]
    devs = [(dev(k), dev(p), dev(h0)) for k, p, h0 in ins]
    alone = [sr.mingru_forward(k=k, p=p, h0=h0) for k, p, h0 in devs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for rep in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                k, p, h0 = devs[i]
                outs[i] = sr.mingru_forward(k=k, p=p, h0=h0)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], alone[i]), (rep, i)
    for i, (k, p, h0) in enumerate(ins):
        assert scan_err(host64(outs[i]), k, p, h0) < TOL_F32
