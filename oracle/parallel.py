"""The oracle run over slices of channels in worker processes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every (batch row, channel) of the scans is its own sequential recurrence, so
the oracle can evaluate disjoint slices of channels in separate processes and
get exactly what one process would: each worker calls the same oracle
functions (``mingru.scan``, ``mingru.scan_terms``, ``metrics``, ...) on its
slice, with no other arithmetic.  This is how the full-size workloads are
checked element by element, and how the CPU baseline uses the host's cores.

Arrays travel through POSIX shared memory; workers are started with the
"spawn" method, so they are fresh interpreters that import NumPy and this
package only (never torch, never the GPU).
"""

from __future__ import annotations

import importlib
import multiprocessing as mp
import os
import time
from multiprocessing import shared_memory

import numpy as np

from . import metrics, mingru

# At most this many worker processes (the host's cores, capped).
MAX_WORKERS = 16

_ARRAYS = {}
_SHMS = []


def default_workers() -> int:
    return max(1, min(os.cpu_count() or 1, MAX_WORKERS))


def _attach(specs):
    for name, (shm_name, shape, dtype) in specs.items():
        shm = shared_memory.SharedMemory(name=shm_name)
        _SHMS.append(shm)
        _ARRAYS[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)


def _run(job):
    module, fn, sl = job
    return getattr(importlib.import_module(module), fn)(_ARRAYS, sl)


def channel_slices(B: int, D: int, width: int):
    """(b, d0, d1) for every batch row and run of `width` channels."""
    return [(b, d0, min(d0 + width, D)) for b in range(B) for d0 in range(0, D, width)]


def _can_spawn() -> bool:
    # Spawned workers re-import the parent's main module by its file; a
    # parent run from stdin or -c has none, and its workers could not start.
    import sys
    path = getattr(sys.modules.get("__main__"), "__file__", None)
    return path is not None and os.path.isfile(path)


def map_slices(task, arrays: dict, slices, workers: int | None = None, timeout: float = 900.0):
    """Calls task(arrays, slice) for every slice in worker processes and
    returns the results in slice order.  `task` is a module-level function
    (referred to by module and name in the workers); `arrays` maps names to
    NumPy arrays, which the workers see read-only through shared memory.
    With one worker, or a parent whose main module has no file, the slices
    run in this process.  A pool that has not finished after `timeout`
    seconds raises TimeoutError."""
    workers = workers or default_workers()
    if workers == 1 or not _can_spawn():
        return [task(arrays, sl) for sl in slices]
    shms, specs = [], {}
    try:
        for name, a in arrays.items():
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
            shms.append(shm)
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            specs[name] = (shm.name, a.shape, a.dtype.str)
        ctx = mp.get_context("spawn")
        jobs = [(task.__module__, task.__name__, sl) for sl in slices]
        pool = ctx.Pool(workers, initializer=_attach, initargs=(specs,))
        try:
            out = pool.map_async(_run, jobs, chunksize=1).get(timeout)
        except BaseException:
            pool.terminate()
            pool.join()
            raise
        # The workers are let finish and exit on their own rather than being
        # sent SIGTERM (what leaving a `with Pool` block does): a process
        # tool preloaded into them (a profiler) may not survive that signal
        # cleanly, and the parent would then wait for them forever.
        pool.close()
        pool.join()
        return out
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()


# ------------------------------------------------------------ minGRU scan

def _slice64(arrays, name, sl):
    b, d0, d1 = sl
    a = arrays[name]
    return np.asarray(a[b:b + 1, ..., d0:d1], dtype=np.float64)


def scan_slice_time(arrays, sl):
    """The oracle's sequential scan on one slice; returns (seconds, elements)."""
    k, p = _slice64(arrays, "k", sl), _slice64(arrays, "p", sl)
    h0 = _slice64(arrays, "h0", sl) if "h0" in arrays else None
    t0 = time.perf_counter()
    mingru.scan(k, p, h0)
    return time.perf_counter() - t0, k.size


def scan_slice_error(arrays, sl):
    """Max conditioned error of arrays["got"] on one slice against the oracle."""
    k, p = _slice64(arrays, "k", sl), _slice64(arrays, "p", sl)
    h0 = _slice64(arrays, "h0", sl) if "h0" in arrays else None
    ref = mingru.scan(k, p, h0)
    carry, inp = mingru.scan_terms(k, p, h0)
    return metrics.h_rel_err(_slice64(arrays, "got", sl), ref, carry, inp)


def mingru_scan_timed(k, p, h0=None, workers: int | None = None, width: int = 64):
    """Runs the sequential oracle on every channel of [B, T, D] inputs and
    times it: returns dict(wall_s, workers, elements)."""
    workers = workers or default_workers()
    arrays = {"k": k, "p": p}
    if h0 is not None:
        arrays["h0"] = h0
    B, _, D = k.shape
    t0 = time.perf_counter()
    res = map_slices(scan_slice_time, arrays, channel_slices(B, D, width), workers)
    wall = time.perf_counter() - t0
    return dict(wall_s=wall, workers=workers, elements=int(sum(n for _, n in res)),
                worker_scan_s=float(sum(s for s, _ in res)))


def mingru_scan_error(k, p, h0, got, workers: int | None = None, width: int = 64) -> float:
    """Max conditioned error of `got` [B, T, D] against the oracle, every
    element of every channel."""
    arrays = {"k": k, "p": p, "got": got}
    if h0 is not None:
        arrays["h0"] = h0
    B, _, D = k.shape
    return max(map_slices(scan_slice_error, arrays, channel_slices(B, D, width), workers))
