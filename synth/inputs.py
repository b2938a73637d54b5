"""Seeded input generators and the five workload shapes.

Every tensor draws from ``numpy.random.default_rng([2026, seed, tensor_id])``
or, for a [B, T, D] sequence tensor, from one generator per block of
``T_BLOCK`` time steps, ``default_rng([2026, seed, tensor_id, tb])`` (``seed`` the
workload's number in ``CONFIGS``), so that any
slice along T can be regenerated without drawing the whole tensor.  Values are
drawn in float64 and rounded to float32 (round to nearest even); the bf16
inputs are rounded once more, float32 -> bf16, again to nearest even.  The
same rounded values feed the GPU library and the oracle.

Large workloads whose host copy would be too heavy to draw in NumPy use
``device_normal`` / ``device_uniform``: a seeded ``torch.Generator`` on the
device.  Those values differ from the NumPy ones but follow the same
distributions, and the oracle reads back whatever slice it checks.

The shapes follow the pages' usage examples: a minGRU layer of width 512 on a
(2, 1024, 512) batch (minGRU-pytorch profile, guide "Install and apply the
minGRU layer") and a MinMax hidden state of d_state = 192 (minmaxrnc,
"Custom configuration").
"""

from __future__ import annotations

import numpy as np
import torch

SEED_ROOT = 2026
T_BLOCK = 512

TENSOR_IDS = {
    "x": 0,
    "W_in": 1,
    "W_out": 2,
    "h0": 3,
    "k": 4,
    "p": 5,
    "r": 6,
    "s": 7,
    "x0": 8,
    "decay_rate": 9,
    "delta_t": 10,
}

# The five workloads, named by what they are and their sizes.  ``seed`` is
# the workload's component of every seed drawn for it.  "N(0, 1/D)" names a
# variance, so the standard deviation is D ** -0.5.
LAYER_TINY = "layer_b2_t64_d16_fp32"
LAYER = "layer_b2_t1024_d512_fp32"
SCAN = "scan_b8_t65536_d1024_bf16"
STEP = "step_b256_d2048_fp32"
MINMAX = "minmax_b8_t32768_d192_fp32"

CONFIGS = {
    LAYER_TINY: dict(seed=1, kind="layer", B=2, T=64, D=16, dtype="f32",
                     w_std=16 ** -0.5, h0=False),
    LAYER: dict(seed=2, kind="layer", B=2, T=1024, D=512, dtype="f32",
                w_std=512 ** -0.5, h0=False),
    SCAN: dict(seed=3, kind="scan", B=8, T=65536, D=1024, dtype="bf16",
               k_mean=-4.0, k_std=1.0, p_mean=0.0, p_std=1.0, h0=True),
    STEP: dict(seed=4, kind="step", B=256, D=2048, T_prefill=512, steps=4096,
               dtype="f32", w_std=2048 ** -0.5),
    MINMAX: dict(seed=5, kind="minmax", B=8, T=32768, D=192, dtype="f32"),
}
for _name, _entry in CONFIGS.items():
    _entry["name"] = _name


def _seed(workload: str) -> int:
    return CONFIGS[workload]["seed"]


def _rng(workload: str, name: str, tb: int | None = None) -> np.random.Generator:
    key = [SEED_ROOT, _seed(workload), TENSOR_IDS[name]]
    if tb is not None:
        key.append(int(tb))
    return np.random.default_rng(key)


def bf16_round(a: np.ndarray) -> torch.Tensor:
    """float32 array -> bf16 tensor, round to nearest even (torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _no_negative_zero(a: np.ndarray) -> np.ndarray:
    # A drawn -0.0 becomes +0.0 so that min/max ties never hinge on the sign
    # of zero.
    a[a == 0] = 0.0
    return a


def normal_bt(workload: str, name: str, B: int, T: int, D: int, mean: float = 0.0,
              std: float = 1.0, t0: int = 0) -> np.ndarray:
    """float32 [B, T, D] sequence tensor ~ N(mean, std^2), drawn per T-block.

    ``t0`` must be a multiple of T_BLOCK; the slice [t0, t0 + T) is returned.
    """
    if t0 % T_BLOCK:
        raise ValueError("t0 must be a multiple of T_BLOCK")
    out = np.empty((B, T, D), dtype=np.float32)
    tb0 = t0 // T_BLOCK
    nb = -(-T // T_BLOCK)
    for i in range(nb):
        lo = i * T_BLOCK
        n = min(T_BLOCK, T - lo)
        blk = _rng(workload, name, tb0 + i).standard_normal((B, T_BLOCK, D))
        out[:, lo:lo + n, :] = (mean + std * blk[:, :n, :]).astype(np.float32)
    return out


def uniform_bt(workload: str, name: str, B: int, T: int, D: int, lo: float,
               hi: float, t0: int = 0) -> np.ndarray:
    """float32 [B, T, D] ~ U(lo, hi) per T-block, no negative zeros."""
    if t0 % T_BLOCK:
        raise ValueError("t0 must be a multiple of T_BLOCK")
    out = np.empty((B, T, D), dtype=np.float32)
    tb0 = t0 // T_BLOCK
    nb = -(-T // T_BLOCK)
    for i in range(nb):
        a = i * T_BLOCK
        n = min(T_BLOCK, T - a)
        blk = _rng(workload, name, tb0 + i).uniform(lo, hi, (B, T_BLOCK, D))
        out[:, a:a + n, :] = blk[:, :n, :].astype(np.float32)
    return _no_negative_zero(out)


def normal_mat(workload: str, name: str, rows: int, cols: int, std: float) -> np.ndarray:
    """float32 weight matrix ~ N(0, std^2)."""
    return (std * _rng(workload, name).standard_normal((rows, cols))).astype(np.float32)


def normal_vec(workload: str, name: str, B: int, D: int, mean: float = 0.0,
               std: float = 1.0) -> np.ndarray:
    """float32 [B, D] state ~ N(mean, std^2)."""
    return (mean + std * _rng(workload, name).standard_normal((B, D))).astype(np.float32)


def uniform_vec(workload: str, name: str, B: int, D: int, lo: float, hi: float) -> np.ndarray:
    return _no_negative_zero(_rng(workload, name).uniform(lo, hi, (B, D)).astype(np.float32))


def decay_rates(workload: str, D: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """float32 [D] per-channel decay rates, log-uniform on [lo, hi] (time
    constants from 1/hi to 1/lo tokens)."""
    u = _rng(workload, "decay_rate").uniform(np.log10(lo), np.log10(hi), D)
    return (10.0 ** u).astype(np.float32)


def gaps(workload: str, B: int, T: int, mean: float = 1.0, p_huge: float = 1e-3,
         huge: float = 1e6, t0: int = 0) -> np.ndarray:
    """float32 [B, T] gaps preceding each token, drawn per T-block: exponential
    with the given mean (irregular event times), except that a fraction
    ``p_huge`` of them is ``huge`` (long silences; with rates above
    1e4 / huge they saturate the decay)."""
    if t0 % T_BLOCK:
        raise ValueError("t0 must be a multiple of T_BLOCK")
    out = np.empty((B, T), dtype=np.float32)
    tb0 = t0 // T_BLOCK
    for i in range(-(-T // T_BLOCK)):
        a = i * T_BLOCK
        n = min(T_BLOCK, T - a)
        rng = _rng(workload, "delta_t", tb0 + i)
        blk = rng.exponential(mean, (B, T_BLOCK))
        blk[rng.random((B, T_BLOCK)) < p_huge] = huge
        out[:, a:a + n] = blk[:, :n].astype(np.float32)
    return out


def _torch_gen(workload: str, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(SEED_ROOT * 1_000_003 + _seed(workload) * 1009 + TENSOR_IDS[name])
    return g


def device_normal(workload: str, name: str, shape, mean: float = 0.0, std: float = 1.0,
                  dtype=torch.float32, device="cuda") -> torch.Tensor:
    """Seeded N(mean, std^2) drawn on ``device`` in float32, then cast to dtype."""
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(mean, std, generator=_torch_gen(workload, name, device))
    return t.to(dtype) if dtype != torch.float32 else t


def device_uniform(workload: str, name: str, shape, lo: float, hi: float,
                   device="cuda") -> torch.Tensor:
    """Seeded U(lo, hi) float32 on ``device``, no negative zeros."""
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.uniform_(lo, hi, generator=_torch_gen(workload, name, device))
    return t.masked_fill_(t == 0, 0.0)
