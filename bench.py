#!/usr/bin/env python3
"""Benchmark of the gfx950 minGRU log-space scan (and its sibling paths).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs scan,minmax,decode,...]

One step is one pass of the scan hot path over one batch: the headline
workload is the long-sequence scan B=8, T=65536, D=1024 with bf16 gate logits
k and candidate pre-activations p, an fp32 carried state h0 and fp32 outputs
h and h_T (the fused activation -> log-space coefficient transform, the
in-register / LDS / look-back scan and the apply + store, all in one launch
after a small workspace reset).  Inputs are seeded synthetic tensors drawn on
the GPU and resident in HBM before the timed region.  The printed JSON line
carries:

* value      -- elements (B*T*D) per second over the K timed steps;
* roofline   -- algorithmic bytes per launch (8 B per element plus h0 and
                h_T) over the median launch duration measured with HIP
                events on the launch stream, against the 8 TB/s HBM peak;
                ``traffic`` comes from committed rocprofv3 counter runs when
                they were taken on the current kernel source, else null;
* cpu_baseline -- the fp64 CPU oracle timed on the same workload (every
                channel, by default the whole sequence; --cpu-steps takes a
                prefix), its channels split over worker processes on the
                host's cores (at most 16; ``cores`` says how many);
* parity     -- the largest conditioned relative error of the timed
                run's output against that oracle, over every element of the
                sample, with the bf16-input tolerance;
* legs       -- the other measurements: the MinMax scan, the backward passes
                of both scans, the time-decayed scan and its backward, the
                decode-style step loop with its prefill, the small layers
                (eagerly and replayed from a HIP graph), the MinMax token
                loop, and the read+write streaming ceiling (the faster of
                the device copy and an elementwise kernel with the same
                traffic; roofline.frac_of_copy_ceiling is relative to it).
                Opt-in (name them in --legs): shapes -- one scan call over
                the sweep shapes (both operators, bf16 and fp32 inputs);
                streams -- read-only, write-only and read+write ceilings of
                torch's own kernels on 2 GiB; step_sweep -- the decode
                step's x_t W_in with the update (B=256, D_h=2048) over
                D_in = 64 .. 4096, with a fixed + per-K fit; placement -- the full-size
                backward (plain and decayed) and forward with their large
                tensors carved from one buffer at chosen relative offsets.

The headline scan is measured last, after the other legs, on a GPU already
at its sustained clock: the full-size backward and time-decayed scans run
right before its warm-up (its inputs are generated before them).  Only one GPU is used; --gpus above 1 exits with a
message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("scan elements/s (B·T·D) + achieved HBM GB/s vs peak, "
          "minGRU log-space scan")
HBM_PEAK_GBPS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_b8_t65536_d1024_bf16_traffic.json")
# The scan kernel's sources: the kernel and the engine it instantiates.
SCAN_SOURCES = [os.path.join(ROOT, "scan_linear_rnn_amd", "csrc", f)
                for f in ("scan.hip", "scan_engine.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths=SCAN_SOURCES) -> str:
    """First 16 hex digits of the SHA-256 of the scan kernel's sources, in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def time_launches(torch, fn, steps, warmup):
    """Runs fn `warmup` times, then `steps` times bracketed by synchronisation.
    Returns (wall seconds for the K steps, per-launch ms from HIP events
    recorded on the current stream around each launch)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) for s, e in zip(starts, ends)]


def release_cached(torch):
    """Hands the blocks freed by earlier legs back to the HIP runtime, so that a
    leg's large tensors are fresh allocations, as in a process of its own.
    The backward reads four and writes two tensors of 1-2 GiB at the same
    offsets; how their base addresses fall relative to each other moves its
    time by up to ~9% (the same kernel: 1.77 ms with the six carved from one
    buffer at GiB boundaries, 1.93 ms with each shifted by a further 6 MiB),
    and blocks reused from earlier legs of other shapes had cost the decayed
    backward 13% (2.107 vs 1.867 ms in one process).  Called before a leg
    makes its inputs, so the GPU is busy again (inputs, forward pass,
    warm-up) before its timed launches."""
    torch.cuda.empty_cache()


def all_finite(torch, t):
    """Whether every element of t is finite, from its minimum and maximum
    (NaN and infinities reach them): two reductions, no temporaries of t's
    size, so the GPU does not sit idle behind allocations between legs."""
    lo, hi = torch.aminmax(t)
    return bool(torch.isfinite(lo).item() and torch.isfinite(hi).item())


def median(xs):
    return statistics.median(xs)


def launch_stats(per, alg_bytes, res):
    """Adds the median / min / mean launch time (ms) and the algorithmic bytes
    over the median launch (GB/s, fraction of the 8 TB/s peak) to res."""
    med = median(per)
    res.update(launch_ms_median=med, launch_ms_min=min(per), launch_ms_mean=sum(per) / len(per),
               achieved_GBps=alg_bytes / (med * 1e-3) / 1e9,
               frac_of_hbm_peak=alg_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS)
    return res


def prepare_scan(torch, sr, synth):
    """The headline scan's inputs, outputs and workspace, made ahead of the
    measurements that precede it (so that nothing but its own warm-up sits
    between the last of them and its timed launches)."""
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] scan B={B} T={T} D={D}: generating inputs")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    y = torch.empty((B, T, D), dtype=torch.float32, device="cuda")
    last = torch.empty((B, D), dtype=torch.float32, device="cuda")
    nbytes = sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    return dict(B=B, T=T, D=D, kb=kb, pb=pb, h0=h0, y=y, last=last, ws=ws, nbytes=nbytes)


def leg_scan(torch, sr, synth, steps, warmup, cpu_steps, prep):
    import ctypes
    B, T, D = prep["B"], prep["T"], prep["D"]
    kb, pb, h0, y, last, ws, nbytes = (prep[k] for k in ("kb", "pb", "h0", "y", "last", "ws", "nbytes"))
    lib = sr.raw_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (B, T, 0, D, D, None, None, ctypes.c_void_p(kb.data_ptr()),
            ctypes.c_void_p(pb.data_ptr()), D, sr.SR_BF16, ctypes.c_void_p(h0.data_ptr()), None,
            ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(last.data_ptr()),
            ctypes.c_void_p(ws.data_ptr()), nbytes, stream)

    def step():
        st = lib.mingru_forward(*args)
        if st:
            raise RuntimeError(lib.scanrnn_last_error().decode())

    log(f"[bench] scan: {warmup} warmup + {steps} timed steps")
    wall, per = time_launches(torch, step, steps, warmup)
    if sr.workspace_status(ws) != 0:
        raise RuntimeError("the scan reported a look-back time-out or an out-of-range gate")
    if not all_finite(torch, y):
        raise RuntimeError("non-finite scan output")
    n = B * T * D
    alg_bytes = n * (2 + 2 + 4) + 2 * B * D * 4
    med = median(per)
    ach = alg_bytes / (med * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == source_hash():
            traffic = tr.get("bytes_per_launch")
    res = dict(
        B=B, T=T, D=D, elements=n, wall_s=wall, ms_per_step=wall / steps * 1e3,
        launch_ms_median=med, launch_ms_min=min(per), launch_ms_mean=sum(per) / len(per),
        value=n / (wall / steps),
        roofline={"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                  "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                  "alg_bytes_per_launch": alg_bytes, "launch_time": "median of the HIP events",
                  "kernel": "chunk_scan_kernel<MinGRUOp, bf16, V=2> (+ workspace reset)"},
    )
    if cpu_steps > 0:
        # The oracle on every channel over the first cpu_steps steps, in
        # worker processes over the host's cores: first timed on its own
        # (the CPU baseline), then run again against the GPU output (parity
        # of every element of that range).
        from oracle import parallel
        ts = min(cpu_steps, T)
        k = kb[:, :ts].float().cpu().numpy()
        p = pb[:, :ts].float().cpu().numpy()
        hh0 = h0.cpu().numpy()
        got = y[:, :ts].cpu().numpy()
        log(f"[bench] scan: CPU oracle on every channel, steps [0, {ts})")
        tm = parallel.mingru_scan_timed(k, p, hh0)
        ns = B * ts * D
        res["cpu_baseline"] = {
            "value": ns / tm["wall_s"], "unit": "elements/s", "cores": tm["workers"],
            "kind": "oracle",
            "sample": f"all {B}x{D} channels, steps [0, {ts}) of T={T} ({ns} elements, "
                      f"{tm['wall_s']:.1f} s wall; NumPy fp64 sequential recurrence, channels "
                      f"split over {tm['workers']} worker processes)",
        }
        log("[bench] scan: parity of every element against the oracle")
        err = parallel.mingru_scan_error(k, p, hh0, got)
        res["parity"] = {"max_conditioned_rel_err": err, "tolerance": 2e-2, "pass": bool(err < 2e-2),
                         "elements_checked": ns,
                         "oracle": "fp64 sequential recurrence on the same bf16 inputs, every element"}
    del kb, pb, y, ws
    prep.clear()
    torch.cuda.empty_cache()
    return res


def leg_minmax(torch, sr, synth, steps, warmup):
    cfg = synth.CONFIGS[synth.MINMAX]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] minmax B={B} T={T} D={D}")
    r = synth.device_uniform(synth.MINMAX, "r", (B, T, D), -1.0, 1.0)
    s = synth.device_uniform(synth.MINMAX, "s", (B, T, D), -1.5, 0.5)
    x0 = synth.device_uniform(synth.MINMAX, "x0", (B, D), -1.0, 1.0)
    out = torch.empty_like(r)
    last = torch.empty((B, D), device="cuda")
    ws = torch.empty(sr.raw_library().minmax_scan_workspace_size(B, T, D), dtype=torch.uint8,
                     device="cuda")

    def step():
        sr.minmax_scan(r, s, x0, return_last=True, workspace=ws, out=out, out_last=last)

    wall, per = time_launches(torch, step, steps, warmup)
    n = B * T * D
    alg = n * 12 + 2 * B * D * 4
    return launch_stats(per, alg, dict(B=B, T=T, D=D, elements_per_s=n / (wall / steps)))


def leg_minmax_step(torch, sr, synth, n_steps):
    """The MinMax neuron one token at a time at the MinMax workload's width
    (B=8, D=192), in place: eagerly and replayed from a HIP graph.  The final
    state is checked bit for bit against the scan over the same tokens."""
    cfg = synth.CONFIGS[synth.MINMAX]
    B, D = cfg["B"], cfg["D"]
    r = synth.device_uniform(synth.MINMAX, "r", (B, n_steps, D), -1.0, 1.0)
    s = synth.device_uniform(synth.MINMAX, "s", (B, n_steps, D), -1.5, 0.5)
    x0 = synth.device_uniform(synth.MINMAX, "x0", (B, D), -1.0, 1.0)
    rs = [r[:, t].contiguous() for t in range(n_steps)]
    ss = [s[:, t].contiguous() for t in range(n_steps)]
    x = torch.empty_like(x0)

    def loop():
        x.copy_(x0)
        for t in range(n_steps):
            sr.minmax_step(rs[t], ss[t], x, x_next=x)

    loop()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    _, last = sr.minmax_scan(r, s, x0, return_last=True)
    exact = bool(torch.equal(x, last))
    res = dict(B=B, D=D, steps=n_steps, step_loop_ms=dt * 1e3, steps_per_s=n_steps / dt,
               matches_scan_bitwise=exact)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    res["graph_step_loop_ms"] = dt * 1e3
    res["graph_steps_per_s"] = n_steps / dt
    res["graph_matches_scan_bitwise"] = bool(torch.equal(x, last))
    del g
    return res


def leg_scan_backward(torch, sr, synth, steps, warmup):
    """Backward of the headline scan: reads k, p (bf16), h, dh (fp32), writes
    dk, dp (fp32): 20 algorithmic bytes per element."""
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] scan backward B={B} T={T} D={D}")
    release_cached(torch)
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    h = sr.mingru_forward(k=kb, p=pb, h0=h0)
    dh = torch.empty_like(h).normal_(0.0, 1.0)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    wall, per = time_launches(
        torch, lambda: sr.mingru_scan_backward(kb, pb, h, dh, h0=h0, workspace=ws), steps, warmup)
    n = B * T * D
    alg = n * 20 + 3 * B * D * 4
    res = launch_stats(per, alg, dict(B=B, T=T, D=D, elements_per_s=n / (wall / steps)))
    del kb, pb, h, dh, ws
    return res


def prepare_scan_decay(torch, sr, synth):
    """The decayed scan's inputs, output and workspace, made ahead (as for
    the headline)."""
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] decayed scan B={B} T={T} D={D}: generating inputs")
    prep = dict(B=B, T=T, D=D)
    prep["kb"] = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"],
                                     torch.bfloat16)
    prep["pb"] = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"],
                                     torch.bfloat16)
    prep["h0"] = synth.device_normal(synth.SCAN, "h0", (B, D))
    prep["rate"] = torch.from_numpy(synth.decay_rates(synth.SCAN, D)).cuda()
    prep["gap"] = torch.from_numpy(synth.gaps(synth.SCAN, B, T)).cuda()
    prep["sat"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    prep["y"] = torch.empty((B, T, D), dtype=torch.float32, device="cuda")
    prep["ws"] = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                             dtype=torch.uint8, device="cuda")
    return prep


def leg_scan_decay(torch, sr, synth, steps, warmup, prep):
    """The headline scan shape with time decay of the carried state: k, p
    (bf16) in, h (fp32) out as in the plain scan, plus one gap per (b, t) and
    one rate per channel: 8 + 4/D algorithmic bytes per element."""
    B, T, D = prep["B"], prep["T"], prep["D"]
    kb, pb, h0, rate, gap, sat, y, ws = (prep[k] for k in
                                        ("kb", "pb", "h0", "rate", "gap", "sat", "y", "ws"))
    log(f"[bench] decayed scan B={B} T={T} D={D}")
    wall, per = time_launches(
        torch, lambda: sr.mingru_forward_decayed(k=kb, p=pb, h0=h0, decay_rate=rate, delta_t=gap,
                                                 saturated=sat, workspace=ws, out=y),
        steps, warmup)
    if sr.workspace_status(ws) != 0 or not all_finite(torch, y):
        raise RuntimeError("decayed scan: look-back expired or non-finite output")
    n = B * T * D
    alg = n * 8 + B * T * 4 + D * 4 + 2 * B * D * 4
    res = launch_stats(per, alg, dict(B=B, T=T, D=D, elements_per_s=n / (wall / steps),
                                      saturated=int(sat.item())))
    # No empty_cache() here: the headline runs next, its buffers already
    # made, and handing gigabytes back to the HIP runtime would leave the GPU idle
    # for milliseconds right before its warm-up.
    del kb, pb, y, ws
    prep.clear()
    return res


def leg_scan_backward_decay(torch, sr, synth, steps, warmup):
    """Backward of the decayed scan at the headline shape: the plain
    backward's 20 bytes per element plus one gap per (b, t) and one rate per
    channel."""
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] decayed scan backward B={B} T={T} D={D}")
    release_cached(torch)
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    rate = torch.from_numpy(synth.decay_rates(synth.SCAN, D)).cuda()
    gap = torch.from_numpy(synth.gaps(synth.SCAN, B, T)).cuda()
    h = sr.mingru_forward_decayed(k=kb, p=pb, h0=h0, decay_rate=rate, delta_t=gap)
    dh = torch.empty_like(h).normal_(0.0, 1.0)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    wall, per = time_launches(
        torch, lambda: sr.mingru_scan_backward_decayed(kb, pb, h, dh, h0=h0, workspace=ws,
                                                       decay_rate=rate, delta_t=gap),
        steps, warmup)
    if sr.workspace_status(ws) != 0:
        raise RuntimeError("decayed scan backward: look-back expired")
    n = B * T * D
    alg = n * 20 + B * T * 4 + D * 4 + 3 * B * D * 4
    res = launch_stats(per, alg, dict(B=B, T=T, D=D, elements_per_s=n / (wall / steps)))
    del kb, pb, h, dh, ws
    return res


def leg_minmax_backward(torch, sr, synth, steps, warmup):
    """Backward of the MinMax scan: reads r, s, x_out, dx, writes dr, ds
    (fp32): 24 algorithmic bytes per element."""
    cfg = synth.CONFIGS[synth.MINMAX]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] minmax backward B={B} T={T} D={D}")
    release_cached(torch)
    r = synth.device_uniform(synth.MINMAX, "r", (B, T, D), -1.0, 1.0)
    s = synth.device_uniform(synth.MINMAX, "s", (B, T, D), -1.5, 0.5)
    x0 = synth.device_uniform(synth.MINMAX, "x0", (B, D), -1.0, 1.0)
    x_out = sr.minmax_scan(r, s, x0)
    dx = torch.empty_like(r).normal_(0.0, 1.0)
    ws = torch.empty(sr.raw_library().minmax_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    wall, per = time_launches(
        torch, lambda: sr.minmax_scan_backward(r, s, x0, x_out, dx, workspace=ws), steps, warmup)
    n = B * T * D
    alg = n * 24 + 2 * B * D * 4
    return launch_stats(per, alg, dict(B=B, T=T, D=D, elements_per_s=n / (wall / steps)))


def leg_decode(torch, sr, synth, n_steps):
    cfg = synth.CONFIGS[synth.STEP]
    B, D, Tp = cfg["B"], cfg["D"], cfg["T_prefill"]
    log(f"[bench] decode: prefill B={B} T={Tp} D={D}, then {n_steps} steps")
    W_in = synth.device_normal(synth.STEP, "W_in", (D, 2 * D), 0.0, cfg["w_std"])
    W_out = synth.device_normal(synth.STEP, "W_out", (D, D), 0.0, cfg["w_std"])
    x = synth.device_normal(synth.STEP, "x", (B, Tp + n_steps, D))
    torch.cuda.synchronize()
    # Prefill (parallel forward over 512 steps), timed on its own.
    y, h = sr.mingru_forward(x[:, :Tp], W_in, W_out=W_out, return_last=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    y, h = sr.mingru_forward(x[:, :Tp], W_in, W_out=W_out, return_last=True)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    prefill_flops = 2.0 * B * Tp * D * (2 * D) + 2.0 * B * Tp * D * D
    xs = [x[:, Tp + t].contiguous() for t in range(n_steps)]
    yt = None
    hh = h.clone()
    for t in range(3):
        yt, hh = sr.mingru_step(xs[t], W_in, W_out, h_prev=hh, h_next=hh)
    hh = h.clone()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(n_steps):
        yt, hh = sr.mingru_step(xs[t], W_in, W_out, h_prev=hh, h_next=hh)
    torch.cuda.synchronize()
    t_steps = time.perf_counter() - t0
    step_flops = 2.0 * B * D * (2 * D) + 2.0 * B * D * D
    return dict(B=B, D=D, prefill_T=Tp, prefill_ms=t_prefill * 1e3,
                prefill_TFLOPs=prefill_flops / t_prefill / 1e12,
                prefill_frac_fp32_mfma=prefill_flops / t_prefill / 1e12 / FP32_MFMA_PEAK_TFLOPS,
                steps=n_steps, steps_per_s=n_steps / t_steps,
                step_us=t_steps / n_steps * 1e6,
                step_TFLOPs=step_flops * n_steps / t_steps / 1e12,
                step_frac_fp32_mfma=step_flops * n_steps / t_steps / 1e12 / FP32_MFMA_PEAK_TFLOPS)


def leg_layer(torch, sr, synth, workload, steps):
    cfg = synth.CONFIGS[workload]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    x = synth.device_normal(workload, "x", (B, T, D))
    W_in = synth.device_normal(workload, "W_in", (D, 2 * D), 0.0, cfg["w_std"])
    W_out = synth.device_normal(workload, "W_out", (D, D), 0.0, cfg["w_std"])
    wall, per = time_launches(torch, lambda: sr.mingru_forward(x, W_in, W_out=W_out), steps, 3)
    res = dict(B=B, T=T, D=D, forward_ms=wall / steps * 1e3, forward_launch_ms=median(per),
               elements_per_s=B * T * D / (wall / steps))
    # The same forward captured once in a HIP graph and replayed (inputs,
    # output and workspace fixed): what a caller bound by launch overhead
    # would run.
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, D, D, D, 1, 1),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty(B, T, D, device="cuda")

    def fwd():
        sr.mingru_forward(x, W_in, W_out=W_out, workspace=ws, out=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    res["graph_forward_ms"] = (time.perf_counter() - t0) / steps * 1e3
    del graph
    xs = [x[:, t].contiguous() for t in range(T)]

    def loop():
        h = None
        for t in range(T):
            _, h = sr.mingru_step(xs[t], W_in, W_out, h_prev=h)
        return h

    loop()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    res["step_loop_ms"] = dt * 1e3
    res["steps_per_s"] = T / dt
    # The same token loop captured once in a HIP graph and replayed (the
    # launch-bound regime: a few tiny kernels per token).
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        loop()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    res["graph_step_loop_ms"] = dt * 1e3
    res["graph_steps_per_s"] = T / dt
    del g
    return res


def leg_copy(torch):
    """Read+write streaming ceiling on 2 GiB (the scan's output size): the
    runtime's device copy and an elementwise kernel with the same traffic
    (one read, one write per element); the faster one is the ceiling."""
    n = 1 << 29
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    copy_ms = median(time_launches(torch, lambda: b.copy_(a), 40, 3)[1])
    elem_ms = median(time_launches(torch, lambda: torch.neg(a, out=b), 40, 3)[1])
    del a, b
    nbytes = 2 * 4 * n
    copy_gbps, elem_gbps = nbytes / (copy_ms * 1e-3) / 1e9, nbytes / (elem_ms * 1e-3) / 1e9
    return dict(bytes_per_copy=nbytes, GBps=max(copy_gbps, elem_gbps), device_copy_GBps=copy_gbps,
                elementwise_GBps=elem_gbps)


# Scan shapes of the sweep table: (B, T, D, input dtype, operator).
SHAPE_SWEEP = [
    (8, 65536, 1024, "bf16", "mingru"), (64, 8192, 1024, "bf16", "mingru"),
    (8, 16384, 4096, "bf16", "mingru"), (32, 65536, 256, "bf16", "mingru"),
    (128, 65536, 64, "bf16", "mingru"), (1, 524288, 1024, "bf16", "mingru"),
    (8, 4096, 1024, "bf16", "mingru"), (8, 1024, 1024, "bf16", "mingru"),
    (2, 1024, 512, "bf16", "mingru"), (8, 16384, 4096, "f32", "mingru"),
    (1, 65536, 1024, "bf16", "mingru"), (8, 65536, 128, "bf16", "mingru"),
    (8, 8192, 1024, "bf16", "mingru"),
    (8, 65536, 1024, "f32", "minmax"), (1, 262144, 192, "f32", "minmax"),
    (1, 32768, 192, "f32", "minmax"),
]


def leg_shapes(torch, sr, synth, steps, warmup):
    """One scan call (workspace reset included) over the sweep shapes: median
    of the HIP events, and the algorithmic bytes over it (minGRU: k, p in,
    h out; MinMax: r, s in, x out; plus h0 and h_T)."""
    lib = sr.raw_library()
    res = {}
    for B, T, D, dt, op in SHAPE_SWEEP:
        tag = f"{op}_{B}x{T}x{D}_{dt}"
        log(f"[bench] shapes: {tag}")
        dtype = torch.bfloat16 if dt == "bf16" else torch.float32
        esz = 2 if dt == "bf16" else 4
        if op == "mingru":
            cfg = synth.CONFIGS[synth.SCAN]
            a = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], dtype)
            b = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], dtype)
            h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
            ws = torch.empty(lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                             dtype=torch.uint8, device="cuda")
            fn = lambda: sr.mingru_forward(k=a, p=b, h0=h0, workspace=ws)
        else:
            a = synth.device_uniform(synth.MINMAX, "r", (B, T, D), -1.0, 1.0)
            b = synth.device_uniform(synth.MINMAX, "s", (B, T, D), -1.5, 0.5)
            h0 = synth.device_uniform(synth.MINMAX, "x0", (B, D), -1.0, 1.0)
            ws = torch.empty(lib.minmax_scan_workspace_size(B, T, D), dtype=torch.uint8,
                             device="cuda")
            fn = lambda: sr.minmax_scan(a, b, h0, workspace=ws)
        _, per = time_launches(torch, fn, steps, warmup)
        alg = B * T * D * (2 * esz + 4) + 2 * B * D * 4
        med = median(per)
        res[tag] = {"launch_ms_median": med, "launch_ms_min": min(per),
                    "frac_of_hbm_peak": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del a, b, h0, ws
        torch.cuda.empty_cache()
    return res


def leg_step_sweep(torch, sr, synth, steps, warmup):
    """The decode step's first product with the update (x_t W_in, then
    h = h + z (g(p) - h); no output projection) at B=256, D_h=2048 over the
    input width D_in: 32 launches captured in a HIP graph and replayed, so
    that the host's per-call cost does not show; GPU time per launch from HIP
    events around the replays (median over `steps` replays), and a
    least-squares line through the points (fixed cost + cost per 1024 of K),
    whose slope gives the K loop's share of the fp32 matrix peak."""
    cfg = synth.CONFIGS[synth.STEP]
    B, D_h = cfg["B"], cfg["D"]
    res = {}
    xs, ys = [], []
    for D_in in (64, 128, 256, 512, 1024, 2048, 4096):
        log(f"[bench] step sweep: D_in={D_in}")
        W_in = torch.empty((D_in, 2 * D_h), device="cuda").normal_(0.0, D_in ** -0.5)
        x = torch.empty((B, D_in), device="cuda").normal_(0.0, 1.0)
        h = torch.zeros((B, D_h), device="cuda")
        ws = torch.empty(max(sr.raw_library().mingru_step_workspace_size(B, D_in, D_h, D_h), 1),
                         dtype=torch.uint8, device="cuda")
        fn = lambda: sr.mingru_step(x, W_in, None, h_prev=h, h_next=h, workspace=ws)
        per_graph = 32
        for _ in range(3):
            fn()  # the kernels' code loaded before the capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                fn()
        med = median(time_launches(torch, graph.replay, steps, warmup)[1]) / per_graph
        flops = 2.0 * B * D_in * 2 * D_h
        res[f"d_in_{D_in}"] = {"launch_us_median": round(med * 1e3, 2),
                               "frac_fp32_mfma": round(flops / (med * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)}
        xs.append(D_in / 1024.0)
        ys.append(med * 1e3)
        del graph, W_in, x, h, ws
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
    flops_per_1024 = 2.0 * B * 1024 * 2 * D_h
    res["fit"] = {"fixed_us": round(my - slope * mx, 2), "us_per_1024_k": round(slope, 2),
                  "k_loop_frac_fp32_mfma": round(flops_per_1024 / (slope * 1e-6) / 1e12 /
                                                 FP32_MFMA_PEAK_TFLOPS, 4)}
    return res


# Relative placements of the placement leg: each tensor's base moves by this
# many bytes beyond the end of the previous one (0: bases 1-2 GiB apart).
PLACEMENT_SHIFTS = [("packed", 0), ("each_+256B", 256), ("each_+64KiB", 64 << 10),
                    ("each_+2MiB", 2 << 20), ("each_+6MiB", 6 << 20), ("each_+37MiB", 37 << 20)]


def leg_placement(torch, sr, synth, steps, warmup):
    """The config-3-shape backward (plain and decayed) and forward with their
    six (backward) or three (forward) large tensors carved from one buffer:
    every base moved by the same shift past the end of the previous tensor.
    Median of the HIP events per call, through the C ABI."""
    import ctypes
    lib = sr.raw_library()
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    n = B * T * D
    names = ["k", "p", "h", "dh", "dk", "dp"]
    sizes = [2 * n, 2 * n, 4 * n, 4 * n, 4 * n, 4 * n]
    total = sum(sizes) + len(sizes) * max(s for _, s in PLACEMENT_SHIFTS) + 256
    log(f"[bench] placement: one {total / 2**30:.1f} GiB buffer")
    release_cached(torch)
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    dh0 = torch.empty_like(h0)
    last = torch.empty_like(h0)
    rate = torch.from_numpy(synth.decay_rates(synth.SCAN, D)).cuda()
    gap = torch.from_numpy(synth.gaps(synth.SCAN, B, T)).cuda()
    wsb = lib.mingru_scan_backward_workspace_size(B, T, D)
    wsf = lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0)
    ws = torch.empty(max(wsb, wsf), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def check(st):
        if st != 0:
            raise RuntimeError(f"placement leg: status {st}: {sr.raw_library().scanrnn_last_error()}")

    res = {}
    for tag, shift in PLACEMENT_SHIFTS:
        v, off = {}, 0
        for nm, size in zip(names, sizes):
            off += shift
            v[nm] = buf[off:off + size].view(torch.bfloat16 if nm in ("k", "p") else torch.float32)
            v[nm] = v[nm].view(B, T, D)
            off += size
        assert off <= total
        v["k"].normal_(cfg["k_mean"], cfg["k_std"])
        v["p"].normal_(cfg["p_mean"], cfg["p_std"])
        v["dh"].normal_(0.0, 1.0)
        fwd = lambda: check(lib.mingru_forward(B, T, 0, D, D, None, None, P(v["k"]), P(v["p"]), D, 1,
                                               P(h0), None, P(v["h"]), P(last), P(ws), wsf, stream))
        bwd = lambda: check(lib.mingru_scan_backward(B, T, D, P(v["k"]), P(v["p"]), D, 1, P(h0),
                                                     P(v["h"]), P(v["dh"]), None, P(v["dk"]),
                                                     P(v["dp"]), P(dh0), P(ws), wsb, stream))
        dec = lambda: check(lib.mingru_scan_backward_decayed(
            B, T, D, P(v["k"]), P(v["p"]), D, 1, P(rate), P(gap), 0, P(h0), P(v["h"]), P(v["dh"]),
            None, P(v["dk"]), P(v["dp"]), P(dh0), P(ws), wsb, stream))
        fwd()  # h from this layout's inputs
        res[tag] = {
            "shift_bytes": shift,
            "forward_ms_median": median(time_launches(torch, fwd, steps, warmup)[1]),
            "backward_ms_median": median(time_launches(torch, bwd, steps, warmup)[1]),
            "decayed_backward_ms_median": median(time_launches(torch, dec, steps, warmup)[1]),
        }
        log(f"[bench] placement {tag}: {res[tag]}")
    del buf, ws
    torch.cuda.empty_cache()
    return res


def leg_streams(torch):
    """Streaming ceilings on 2 GiB fp32 buffers with torch's own kernels:
    read-only (a sum), write-only (a fill), read + write (copy, and an
    elementwise negation); GB/s over the median launch."""
    n = 1 << 29
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    r = torch.empty((), dtype=torch.float32, device="cuda")
    nb = 4 * n
    out = {}
    for name, fn, nbytes in [("read_sum", lambda: torch.sum(a, 0, out=r), nb),
                             ("write_fill", lambda: b.fill_(2.0), nb),
                             ("copy", lambda: b.copy_(a), 2 * nb),
                             ("elementwise_neg", lambda: torch.neg(a, out=b), 2 * nb)]:
        med = median(time_launches(torch, fn, 40, 3)[1])
        out[name] = {"GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "launch_ms_median": med}
    del a, b
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # A fresh process reaches steady clocks only after a few hundred ms of
    # sustained load (measured: the first ~100 launches run 3-5% slower).
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--legs", default="minmax,minmax_bwd,minmax_step,layer_d512,layer_d16,decode,"
                                      "copy,scan_bwd,scan_decay_bwd,scan_decay,scan",
                    help="measurements to run (they always run in the order of this default)")
    ap.add_argument("--cpu-steps", type=int, default=65536,
                    help="sequence prefix the CPU oracle baseline runs over (0 = skip)")
    ap.add_argument("--decode-steps", type=int, default=4096)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import scan_linear_rnn_amd as sr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    legs = [s.strip() for s in args.legs.split(",") if s.strip()]
    # The runtime loads a kernel's code on its first use (milliseconds each):
    # use the checks' kernels and the full-size scans' kernel variants once
    # now, on small inputs, not between two timed legs (an idle stretch
    # before a leg makes its first launches' clocks overshoot and dip).
    all_finite(torch, torch.zeros(64, device="cuda"))
    kw = torch.zeros((1, 300, 256), dtype=torch.bfloat16, device="cuda")
    hw = torch.zeros((1, 256), device="cuda")
    sr.mingru_forward(k=kw, p=kw, h0=hw)
    sr.mingru_forward_decayed(k=kw, p=kw, h0=hw, decay_rate=torch.zeros(256, device="cuda"),
                              delta_t=torch.zeros((1, 300), device="cuda"))
    torch.cuda.synchronize()
    out = {"metric": METRIC}
    extra = {}
    head = None
    # The headline scan runs last, after the other measurements (the copy
    # ceiling just before it), so that it is timed on a GPU already at its
    # sustained clock rather than in the first milliseconds of the process.
    # Order: the short and launch-bound legs first, then the copy ceiling,
    # then the full-size scans, the headline last.  The inputs of the last
    # two legs (decayed scan, headline) are made before the backward legs,
    # so that no allocation or host-side generation leaves the GPU idle
    # between those timed legs: after an idle stretch of some milliseconds a
    # leg's launches run up to 15% slower for about ten launches (the clocks
    # overshoot and recover).
    if "minmax" in legs:
        extra["minmax_b8_t32768_d192"] = leg_minmax(torch, sr, synth, args.steps, args.warmup)
    if "minmax_bwd" in legs:
        extra["minmax_backward_b8_t32768_d192"] = leg_minmax_backward(torch, sr, synth, args.steps,
                                                                      args.warmup)
    if "minmax_step" in legs:
        extra["minmax_step_b8_d192"] = leg_minmax_step(torch, sr, synth, 4096)
    if "layer_d512" in legs:
        extra["layer_b2_t1024_d512"] = leg_layer(torch, sr, synth, synth.LAYER, 10)
    if "layer_d16" in legs:
        extra["layer_b2_t64_d16"] = leg_layer(torch, sr, synth, synth.LAYER_TINY, 10)
    if "decode" in legs:
        extra["step_b256_d2048"] = leg_decode(torch, sr, synth, args.decode_steps)
    if "shapes" in legs:
        extra["scan_shapes"] = leg_shapes(torch, sr, synth, 20, 5)
    if "streams" in legs:
        extra["stream_ceilings"] = leg_streams(torch)
    if "step_sweep" in legs:
        extra["step_sweep_b256_dh2048"] = leg_step_sweep(torch, sr, synth, 30, 5)
    if "placement" in legs:
        extra["placement_b8_t65536_d1024"] = leg_placement(torch, sr, synth, 40, 60)
    if "copy" in legs:
        extra["copy_ceiling"] = leg_copy(torch)
    prep = prepare_scan(torch, sr, synth) if "scan" in legs else None
    prep_decay = prepare_scan_decay(torch, sr, synth) if "scan_decay" in legs else None
    if "scan_bwd" in legs:
        extra["backward_b8_t65536_d1024"] = leg_scan_backward(torch, sr, synth, args.steps, args.warmup)
    if "scan_decay_bwd" in legs:
        extra["decayed_backward_b8_t65536_d1024"] = leg_scan_backward_decay(
            torch, sr, synth, args.steps, args.warmup)
    if "scan_decay" in legs:
        extra["decayed_b8_t65536_d1024"] = leg_scan_decay(torch, sr, synth, args.steps, args.warmup,
                                                          prep_decay)
    if "scan" in legs:
        head = leg_scan(torch, sr, synth, args.steps, args.warmup, args.cpu_steps, prep)
    if head is not None:
        out.update({
            "value": head["value"], "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "minGRU log-space scan, B=8 T=65536 D=1024, bf16 k/p inputs, "
                                   "fp32 h0/h/h_T", "B": head["B"], "T": head["T"], "D": head["D"],
                       "inputs": "bf16", "parallelism": "single GPU"},
            "roofline": head["roofline"],
        })
        if "cpu_baseline" in head:
            out["cpu_baseline"] = head["cpu_baseline"]
        if "parity" in head:
            out["parity"] = head["parity"]
        extra["scan_launch_ms"] = {"median": head["launch_ms_median"], "min": head["launch_ms_min"],
                                   "mean": head["launch_ms_mean"]}
        if "copy_ceiling" in extra:
            out["roofline"]["frac_of_copy_ceiling"] = round(
                out["roofline"]["achieved"] / extra["copy_ceiling"]["GBps"], 4)
    out["legs"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
