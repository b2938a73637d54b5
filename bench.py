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
                h_T) over the average launch duration measured with HIP
                events on the launch stream, against the 8 TB/s HBM peak;
                ``traffic`` comes from committed rocprofv3 counter runs when
                they were taken on the current kernel source, else null;
* cpu_baseline -- the fp64 CPU oracle timed on a bounded sample of the same
                workload (every channel; by default the whole sequence,
                --cpu-steps takes a prefix);
* legs       -- the other measurements: the MinMax scan, the backward passes
                of both scans, the time-decayed scan and its backward, the
                decode-style step loop with its prefill, the small layers
                (eagerly and replayed from a HIP graph), the MinMax token
                loop, and the read+write streaming ceiling (the faster of
                the device copy and an elementwise kernel with the same
                traffic; roofline.frac_of_copy_ceiling is relative to it).

Only one GPU is used; --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
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
    Returns (wall seconds for the K steps, mean per-launch ms from HIP events
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
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, sum(per) / len(per), min(per)


def leg_scan(torch, sr, synth, steps, warmup, cpu_steps):
    import ctypes
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] scan B={B} T={T} D={D}: generating inputs")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    y = torch.empty((B, T, D), dtype=torch.float32, device="cuda")
    last = torch.empty((B, D), dtype=torch.float32, device="cuda")
    lib = sr.raw_library()
    nbytes = lib.mingru_forward_workspace_size(B, T, 0, D, D, 0, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
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
    wall, mean_ms, min_ms = time_launches(torch, step, steps, warmup)
    if sr.workspace_status(ws) != 0:
        raise RuntimeError("look-back wait expired during the benchmark")
    if not bool(torch.isfinite(y).all()):
        raise RuntimeError("non-finite scan output")
    n = B * T * D
    alg_bytes = n * (2 + 2 + 4) + 2 * B * D * 4
    ach = alg_bytes / (mean_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == source_hash():
            traffic = tr.get("bytes_per_launch")
    res = dict(
        B=B, T=T, D=D, elements=n, wall_s=wall, ms_per_step=wall / steps * 1e3,
        launch_ms_mean=mean_ms, launch_ms_min=min_ms,
        value=n / (wall / steps),
        roofline={"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                  "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic,
                  "alg_bytes_per_launch": alg_bytes,
                  "kernel": "chunk_scan_kernel<MinGRUOp, bf16, V=2> (+ workspace reset)"},
    )
    if cpu_steps > 0:
        log(f"[bench] scan: CPU oracle on every channel, first {cpu_steps} steps")
        from oracle import mingru
        ks = kb[:, :cpu_steps].double().cpu().numpy()
        ps = pb[:, :cpu_steps].double().cpu().numpy()
        hs = h0.double().cpu().numpy()
        t0 = time.perf_counter()
        mingru.scan(ks, ps, hs)
        dt = time.perf_counter() - t0
        ns = B * cpu_steps * D
        res["cpu_baseline"] = {
            "value": ns / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"all {B}x{D} channels, steps [0, {cpu_steps}) of T={T} "
                      f"({ns} elements, {dt:.1f} s; NumPy fp64 sequential loop, one thread)",
        }
    del kb, pb, y, ws
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

    wall, mean_ms, min_ms = time_launches(torch, step, steps, warmup)
    n = B * T * D
    alg = n * 12 + 2 * B * D * 4
    return dict(B=B, T=T, D=D, elements_per_s=n / (wall / steps), launch_ms_mean=mean_ms,
                achieved_GBps=alg / (mean_ms * 1e-3) / 1e9,
                frac_of_hbm_peak=alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)


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
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    h = sr.mingru_forward(k=kb, p=pb, h0=h0)
    dh = torch.empty_like(h).normal_(0.0, 1.0)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    wall, mean_ms, min_ms = time_launches(
        torch, lambda: sr.mingru_scan_backward(kb, pb, h, dh, h0=h0, workspace=ws), steps, warmup)
    n = B * T * D
    alg = n * 20 + 3 * B * D * 4
    res = dict(B=B, T=T, D=D, launch_ms_mean=mean_ms, elements_per_s=n / (wall / steps),
               achieved_GBps=alg / (mean_ms * 1e-3) / 1e9,
               frac_of_hbm_peak=alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
    del kb, pb, h, dh, ws
    torch.cuda.empty_cache()
    return res


def leg_scan_decay(torch, sr, synth, steps, warmup):
    """The headline scan shape with time decay of the carried state: k, p
    (bf16) in, h (fp32) out as in the plain scan, plus one gap per (b, t) and
    one rate per channel: 8 + 4/D algorithmic bytes per element."""
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] decayed scan B={B} T={T} D={D}")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    rate = torch.from_numpy(synth.decay_rates(synth.SCAN, D)).cuda()
    gap = torch.from_numpy(synth.gaps(synth.SCAN, B, T)).cuda()
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty((B, T, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(sr.raw_library().mingru_forward_workspace_size(B, T, 0, D, D, 0, 0),
                     dtype=torch.uint8, device="cuda")
    wall, mean_ms, _ = time_launches(
        torch, lambda: sr.mingru_forward_decayed(k=kb, p=pb, h0=h0, decay_rate=rate, delta_t=gap,
                                                 saturated=sat, workspace=ws, out=y),
        steps, warmup)
    if sr.workspace_status(ws) != 0 or not bool(torch.isfinite(y).all()):
        raise RuntimeError("decayed scan: look-back expired or non-finite output")
    n = B * T * D
    alg = n * 8 + B * T * 4 + D * 4 + 2 * B * D * 4
    res = dict(B=B, T=T, D=D, launch_ms_mean=mean_ms, elements_per_s=n / (wall / steps),
               achieved_GBps=alg / (mean_ms * 1e-3) / 1e9,
               frac_of_hbm_peak=alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               saturated=int(sat.item()))
    del kb, pb, y, ws
    torch.cuda.empty_cache()
    return res


def leg_scan_backward_decay(torch, sr, synth, steps, warmup):
    """Backward of the decayed scan at the headline shape: the plain
    backward's 20 bytes per element plus one gap per (b, t) and one rate per
    channel."""
    cfg = synth.CONFIGS[synth.SCAN]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] decayed scan backward B={B} T={T} D={D}")
    kb = synth.device_normal(synth.SCAN, "k", (B, T, D), cfg["k_mean"], cfg["k_std"], torch.bfloat16)
    pb = synth.device_normal(synth.SCAN, "p", (B, T, D), cfg["p_mean"], cfg["p_std"], torch.bfloat16)
    h0 = synth.device_normal(synth.SCAN, "h0", (B, D))
    rate = torch.from_numpy(synth.decay_rates(synth.SCAN, D)).cuda()
    gap = torch.from_numpy(synth.gaps(synth.SCAN, B, T)).cuda()
    h = sr.mingru_forward_decayed(k=kb, p=pb, h0=h0, decay_rate=rate, delta_t=gap)
    dh = torch.empty_like(h).normal_(0.0, 1.0)
    ws = torch.empty(sr.raw_library().mingru_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    wall, mean_ms, _ = time_launches(
        torch, lambda: sr.mingru_scan_backward_decayed(kb, pb, h, dh, h0=h0, workspace=ws,
                                                       decay_rate=rate, delta_t=gap),
        steps, warmup)
    if sr.workspace_status(ws) != 0:
        raise RuntimeError("decayed scan backward: look-back expired")
    n = B * T * D
    alg = n * 20 + B * T * 4 + D * 4 + 3 * B * D * 4
    res = dict(B=B, T=T, D=D, launch_ms_mean=mean_ms, elements_per_s=n / (wall / steps),
               achieved_GBps=alg / (mean_ms * 1e-3) / 1e9,
               frac_of_hbm_peak=alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
    del kb, pb, h, dh, ws
    torch.cuda.empty_cache()
    return res


def leg_minmax_backward(torch, sr, synth, steps, warmup):
    """Backward of the MinMax scan: reads r, s, x_out, dx, writes dr, ds
    (fp32): 24 algorithmic bytes per element."""
    cfg = synth.CONFIGS[synth.MINMAX]
    B, T, D = cfg["B"], cfg["T"], cfg["D"]
    log(f"[bench] minmax backward B={B} T={T} D={D}")
    r = synth.device_uniform(synth.MINMAX, "r", (B, T, D), -1.0, 1.0)
    s = synth.device_uniform(synth.MINMAX, "s", (B, T, D), -1.5, 0.5)
    x0 = synth.device_uniform(synth.MINMAX, "x0", (B, D), -1.0, 1.0)
    x_out = sr.minmax_scan(r, s, x0)
    dx = torch.empty_like(r).normal_(0.0, 1.0)
    ws = torch.empty(sr.raw_library().minmax_scan_backward_workspace_size(B, T, D),
                     dtype=torch.uint8, device="cuda")
    wall, mean_ms, _ = time_launches(
        torch, lambda: sr.minmax_scan_backward(r, s, x0, x_out, dx, workspace=ws), steps, warmup)
    n = B * T * D
    alg = n * 24 + 2 * B * D * 4
    return dict(B=B, T=T, D=D, launch_ms_mean=mean_ms, elements_per_s=n / (wall / steps),
                achieved_GBps=alg / (mean_ms * 1e-3) / 1e9,
                frac_of_hbm_peak=alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)


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
    wall, mean_ms, _ = time_launches(torch, lambda: sr.mingru_forward(x, W_in, W_out=W_out),
                                     steps, 3)
    res = dict(B=B, T=T, D=D, forward_ms=wall / steps * 1e3, forward_launch_ms=mean_ms,
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
    _, copy_ms, _ = time_launches(torch, lambda: b.copy_(a), 10, 3)
    _, elem_ms, _ = time_launches(torch, lambda: torch.neg(a, out=b), 10, 3)
    del a, b
    torch.cuda.empty_cache()
    nbytes = 2 * 4 * n
    copy_gbps, elem_gbps = nbytes / (copy_ms * 1e-3) / 1e9, nbytes / (elem_ms * 1e-3) / 1e9
    return dict(bytes_per_copy=nbytes, GBps=max(copy_gbps, elem_gbps), device_copy_GBps=copy_gbps,
                elementwise_GBps=elem_gbps)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # A fresh process reaches steady clocks only after a few hundred ms of
    # sustained load (measured: the first ~100 launches run 3-5% slower).
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--legs", default="scan,minmax,scan_bwd,minmax_bwd,scan_decay,scan_decay_bwd,"
                                      "decode,layer_d512,layer_d16,minmax_step,copy")
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
    out = {"metric": METRIC}
    extra = {}
    head = None
    if "scan" in legs:
        head = leg_scan(torch, sr, synth, args.steps, args.warmup, args.cpu_steps)
    if "copy" in legs:
        extra["copy_ceiling"] = leg_copy(torch)
    if "minmax" in legs:
        extra["minmax_b8_t32768_d192"] = leg_minmax(torch, sr, synth, args.steps, args.warmup)
    if "scan_bwd" in legs:
        extra["backward_b8_t65536_d1024"] = leg_scan_backward(torch, sr, synth, args.steps, args.warmup)
    if "minmax_bwd" in legs:
        extra["minmax_backward_b8_t32768_d192"] = leg_minmax_backward(torch, sr, synth, args.steps,
                                                                  args.warmup)
    if "scan_decay" in legs:
        extra["decayed_b8_t65536_d1024"] = leg_scan_decay(torch, sr, synth, args.steps, args.warmup)
    if "scan_decay_bwd" in legs:
        extra["decayed_backward_b8_t65536_d1024"] = leg_scan_backward_decay(
            torch, sr, synth, args.steps, args.warmup)
    if "layer_d512" in legs:
        extra["layer_b2_t1024_d512"] = leg_layer(torch, sr, synth, synth.LAYER, 10)
    if "layer_d16" in legs:
        extra["layer_b2_t64_d16"] = leg_layer(torch, sr, synth, synth.LAYER_TINY, 10)
    if "decode" in legs:
        extra["step_b256_d2048"] = leg_decode(torch, sr, synth, args.decode_steps)
    if "minmax_step" in legs:
        extra["minmax_step_b8_d192"] = leg_minmax_step(torch, sr, synth, 4096)
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
        extra["scan_launch_ms_mean"] = head["launch_ms_mean"]
        extra["scan_launch_ms_min"] = head["launch_ms_min"]
        if "copy_ceiling" in extra:
            out["roofline"]["frac_of_copy_ceiling"] = round(
                out["roofline"]["achieved"] / extra["copy_ceiling"]["GBps"], 4)
    out["legs"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
