"""Python binding of libscanrnn.so, the gfx950 minGRU / MinMax scan library.

The calls carry the C ABI's names (include/scanrnn.h) and only marshal
arguments: they check devices, dtypes and shapes, allocate outputs and the
workspace through PyTorch's caching allocator, and pass raw device pointers
and PyTorch's current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no other code path.
If the shared library is missing the import fails loudly.

    from scan_linear_rnn_amd import MinGRU, mingru_forward, mingru_step, minmax_scan

The layer object follows the minGRU profile's usage (guide "Install and apply
the minGRU layer": a layer of width 512 applied to a (2, 1024, 512) batch
returns the same shape; guide "Process a sequence sequentially": per token,
pass the previous hidden state -- None at first -- with
return_next_prev_hidden=True and keep the returned state).

mingru_scan is the one convenience beyond the C names: the scan-only
forward and its backward kernel in a torch.autograd.Function, so that a
caller can train through the scan (autograd only records the call).
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MinGRU",
    "mingru_scan",
    "mingru_forward",
    "mingru_forward_decayed",
    "mingru_step",
    "mingru_step_decayed",
    "minmax_scan",
    "mingru_scan_backward",
    "mingru_scan_backward_decayed",
    "minmax_scan_backward",
    "library_path",
    "ScanRNNError",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SCANRNN_LIBRARY names another build of the same library to load instead of
# the in-tree one (the host-sanitizer build of build.py uses it).
_LIB_PATH = os.environ.get("SCANRNN_LIBRARY") or os.path.join(_PKG, "libscanrnn.so")

SR_OK = 0
SR_ERR_INVALID_ARGUMENT = 1
SR_ERR_UNSUPPORTED = 2
SR_ERR_WORKSPACE_TOO_SMALL = 3
SR_ERR_HIP = 4
SR_ERR_LOOKBACK_TIMEOUT = 5
SR_ERR_GATE_RANGE = 6
SR_F32 = 0
SR_BF16 = 1
LOOKBACK_SPIN_LIMIT = 1 << 20  # SCANRNN_LOOKBACK_SPIN_LIMIT

EXPORTED = (
    "mingru_forward_workspace_size",
    "mingru_forward",
    "mingru_step_workspace_size",
    "mingru_step",
    "mingru_forward_decayed",
    "mingru_step_decayed",
    "minmax_scan_workspace_size",
    "minmax_scan",
    "minmax_step",
    "mingru_scan_backward_workspace_size",
    "mingru_scan_backward",
    "mingru_scan_backward_decayed",
    "minmax_scan_backward_workspace_size",
    "minmax_scan_backward",
    "mingru_scan_noalloc_max_workspace",
    "mingru_scan_noalloc",
    "scanrnn_last_error",
    "scanrnn_set_lookback_spin_limit",
    "scanrnn_workspace_status",
    "scanrnn_version",
)


class ScanRNNError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python scan_linear_rnn_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, sz, vp, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    lib.mingru_forward_workspace_size.restype = sz
    lib.mingru_forward_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32]
    lib.mingru_forward.restype = i32
    lib.mingru_forward.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, i64, i32, vp, vp,
                                   vp, vp, vp, sz, vp]
    lib.mingru_step_workspace_size.restype = sz
    lib.mingru_step_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.mingru_step.restype = i32
    lib.mingru_step.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mingru_forward_decayed.restype = i32
    lib.mingru_forward_decayed.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, i64, i32,
                                           vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mingru_step_decayed.restype = i32
    lib.mingru_step_decayed.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                        vp, vp, sz, vp]
    lib.minmax_scan_workspace_size.restype = sz
    lib.minmax_scan_workspace_size.argtypes = [i64, i64, i64]
    lib.minmax_scan.restype = i32
    lib.minmax_scan.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.minmax_step.restype = i32
    lib.minmax_step.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    lib.mingru_scan_backward_workspace_size.restype = sz
    lib.mingru_scan_backward_workspace_size.argtypes = [i64, i64, i64]
    lib.minmax_scan_backward_workspace_size.restype = sz
    lib.minmax_scan_backward_workspace_size.argtypes = [i64, i64, i64]
    lib.mingru_scan_backward.restype = i32
    lib.mingru_scan_backward.argtypes = [i64, i64, i64, vp, vp, i64, i32, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp]
    lib.mingru_scan_backward_decayed.restype = i32
    lib.mingru_scan_backward_decayed.argtypes = [i64, i64, i64, vp, vp, i64, i32, vp, vp, i32, vp,
                                                 vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.minmax_scan_backward.restype = i32
    lib.minmax_scan_backward.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp]
    lib.mingru_scan_noalloc_max_workspace.restype = sz
    lib.mingru_scan_noalloc_max_workspace.argtypes = []
    lib.mingru_scan_noalloc.restype = i32
    lib.mingru_scan_noalloc.argtypes = [i64, i64, i64, vp, vp, i64, i32, vp, vp, vp, vp]
    lib.scanrnn_last_error.restype = ctypes.c_char_p
    lib.scanrnn_last_error.argtypes = []
    lib.scanrnn_set_lookback_spin_limit.restype = i32
    lib.scanrnn_set_lookback_spin_limit.argtypes = [ctypes.c_uint32]
    lib.scanrnn_workspace_status.restype = i32
    lib.scanrnn_workspace_status.argtypes = [vp, vp]
    lib.scanrnn_version.restype = ctypes.c_char_p
    lib.scanrnn_version.argtypes = []
    return lib


_lib = _load()


def raw_library() -> ctypes.CDLL:
    """The loaded ctypes library (for ABI-level tests)."""
    return _lib


def _check(fn: str, status: int) -> None:
    if status != SR_OK:
        msg = _lib.scanrnn_last_error().decode(errors="replace")
        raise ScanRNNError(fn, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_stand_ins = {}


def _operand(t):
    """Pointer of an optional weight that is present.  The C calls read NULL
    as "absent" (no projection), so a present weight with no elements (D_in
    or D_h of 0), whose tensor has no storage, is passed as a valid non-NULL
    address that the library never dereferences."""
    if t is None:
        return None
    if t.numel() > 0:
        return ctypes.c_void_p(t.data_ptr())
    dev = t.device
    if dev not in _stand_ins:
        _stand_ins[dev] = torch.zeros(4, dtype=torch.float32, device=dev)
    return ctypes.c_void_p(_stand_ins[dev].data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=torch.float32, ndim=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.contiguous()


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _use_workspace(workspace, nbytes: int, device) -> torch.Tensor:
    """The caller's workspace (checked), or a fresh one when none is given."""
    if workspace is None:
        return _workspace(nbytes, device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a torch.uint8 tensor")
    if workspace.device != torch.device(device) or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {nbytes} needed")
    return workspace


def mingru_forward(x=None, W_in=None, *, k=None, p=None, h0=None, W_out=None,
                   return_last=False, workspace=None, out=None, out_last=None):
    """Parallel mode over a whole sequence.

    Either ``x`` [B,T,D_in] with ``W_in`` [D_in, 2*D_h], or the pre-projected
    ``k``, ``p`` ([B,T,D_h], fp32 or bf16, or two halves of one [B,T,2*D_h]
    buffer).  ``h0`` [B,D_h] is the carried state (None = zero), ``W_out``
    [D_h, D_out] the output projection (None = identity).  Returns y
    [B,T,D_out] fp32, and h_T [B,D_h] when ``return_last``.
    """
    return _forward(x, W_in, k, p, h0, W_out, return_last, workspace, out, out_last, None)


def mingru_forward_decayed(x=None, W_in=None, *, decay_rate, delta_t, log1p_delta=False,
                           saturated=None, k=None, p=None, h0=None, W_out=None,
                           return_last=False, workspace=None, out=None, out_last=None):
    """``mingru_forward`` with time decay of the carried state: before token
    t's write, h is scaled by exp(-min(decay_rate_d * gap_t, 1e4)), gap_t =
    delta_t[b, t] (log1p of it with ``log1p_delta``).

    ``decay_rate`` [D_h] fp32 (>= 0), ``delta_t`` [B,T] fp32 (>= 0, finite).
    ``saturated``: an optional int32 GPU tensor of one element that the call
    sets to 1 (never clears) when some rate * gap exceeds 1e4.
    """
    return _forward(x, W_in, k, p, h0, W_out, return_last, workspace, out, out_last,
                    (decay_rate, delta_t, log1p_delta, saturated))


def _decay_args(decay, D_h, gap_shape, device):
    rate, gap, log1p, sat = decay
    rate = _dev(rate, "decay_rate", shape=(D_h,))
    gap = _dev(gap, "delta_t", shape=gap_shape)
    if sat is not None:
        sat = _dev(sat, "saturated", dtype=torch.int32)
        if sat.numel() < 1 or not sat.is_contiguous():
            raise ValueError("saturated must be a contiguous int32 tensor of at least one element")
    for t, name in ((rate, "decay_rate"), (gap, "delta_t"), (sat, "saturated")):
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be on {device}")
    return rate, gap, int(bool(log1p)), sat


def _forward(x, W_in, k, p, h0, W_out, return_last, workspace, out, out_last, decay):
    if W_in is not None:
        x = _dev(x, "x", ndim=3)
        W_in = _dev(W_in, "W_in", ndim=2)
        B, T, D_in = x.shape
        if W_in.shape[0] != D_in or W_in.shape[1] % 2:
            raise ValueError(f"W_in must be [{D_in}, 2*D_h] (got {tuple(W_in.shape)})")
        D_h = W_in.shape[1] // 2
        device = x.device
        kk = pp = None
        ld_kp, kp_dtype = 0, SR_F32
    else:
        if x is not None:
            raise ValueError("pass either x with W_in, or k and p")
        if k is None or p is None:
            raise ValueError("k and p are required when W_in is None")
        if k.dtype not in (torch.float32, torch.bfloat16) or p.dtype != k.dtype:
            raise TypeError("k and p must both be float32 or both bfloat16")
        if k.device.type != "cuda" or p.device != k.device:
            raise ValueError("k and p must be on the same GPU")
        if k.dim() != 3 or p.shape != k.shape:
            raise ValueError("k and p must be [B,T,D_h] of the same shape")
        B, T, D_h = k.shape
        D_in = 0
        device = k.device
        # Rows may be strided (two halves of one buffer); the feature dim must
        # be unit-stride and both must share one row stride.
        if (k.stride(2) != 1 or p.stride(2) != 1 or k.stride(0) != T * k.stride(1)
                or p.stride(1) != k.stride(1) or p.stride(0) != k.stride(0)):
            k = k.contiguous()
            p = p.contiguous()
        ld_kp = k.stride(1)
        kp_dtype = SR_BF16 if k.dtype == torch.bfloat16 else SR_F32
        kk, pp = k, p
    if h0 is not None:
        h0 = _dev(h0, "h0", shape=(B, D_h))
    if W_out is not None:
        W_out = _dev(W_out, "W_out", ndim=2)
        if W_out.shape[0] != D_h:
            raise ValueError(f"W_out must be [{D_h}, D_out] (got {tuple(W_out.shape)})")
        D_out = W_out.shape[1]
    else:
        D_out = D_h
    if out is not None:
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        y = _dev(out, "out", shape=(B, T, D_out))
    else:
        y = torch.empty((B, T, D_out), dtype=torch.float32, device=device)
    h_last = None
    if return_last:
        if out_last is not None:
            if not out_last.is_contiguous():
                raise ValueError("out_last must be contiguous")
            h_last = _dev(out_last, "out_last", shape=(B, D_h))
        else:
            h_last = torch.empty((B, D_h), dtype=torch.float32, device=device)
    nbytes = _lib.mingru_forward_workspace_size(B, T, D_in, D_h, D_out, int(W_in is not None),
                                                int(W_out is not None))
    ws = _use_workspace(workspace, nbytes, device)
    if decay is None:
        st = _lib.mingru_forward(B, T, D_in, D_h, D_out, _ptr(x if W_in is not None else None),
                                 _operand(W_in), _ptr(kk), _ptr(pp), ld_kp, kp_dtype, _ptr(h0),
                                 _operand(W_out), _ptr(y), _ptr(h_last), _ptr(ws), ws.numel(),
                                 _stream(device))
        _check("mingru_forward", st)
    else:
        rate, gap, log1p, sat = _decay_args(decay, D_h, (B, T), device)
        st = _lib.mingru_forward_decayed(B, T, D_in, D_h, D_out,
                                         _ptr(x if W_in is not None else None), _operand(W_in),
                                         _ptr(kk), _ptr(pp), ld_kp, kp_dtype, _ptr(rate),
                                         _ptr(gap), log1p, _ptr(sat), _ptr(h0), _operand(W_out),
                                         _ptr(y), _ptr(h_last), _ptr(ws), ws.numel(),
                                         _stream(device))
        _check("mingru_forward_decayed", st)
    return (y, h_last) if return_last else y


def mingru_step(x_t, W_in, W_out=None, h_prev=None, h_next=None, workspace=None):
    """Sequential mode, one token: x_t [B,D_in] -> (y_t [B,D_out], h_t [B,D_h]).

    ``h_prev`` None is the zero state.  ``h_next`` may be given (it may be the
    same tensor as ``h_prev``) to avoid an allocation.  Without ``W_out`` the
    output is the new hidden state itself (the same tensor is returned twice).
    """
    return _step(x_t, W_in, W_out, h_prev, h_next, workspace, None)


def mingru_step_decayed(x_t, W_in, W_out=None, h_prev=None, h_next=None, workspace=None, *,
                        decay_rate, delta_t, log1p_delta=False, saturated=None):
    """``mingru_step`` with time decay: ``delta_t`` [B] is the gap preceding
    this token (see ``mingru_forward_decayed``)."""
    return _step(x_t, W_in, W_out, h_prev, h_next, workspace,
                 (decay_rate, delta_t, log1p_delta, saturated))


def _step(x_t, W_in, W_out, h_prev, h_next, workspace, decay):
    x_t = _dev(x_t, "x_t", ndim=2)
    W_in = _dev(W_in, "W_in", ndim=2)
    B, D_in = x_t.shape
    if W_in.shape[0] != D_in or W_in.shape[1] % 2:
        raise ValueError(f"W_in must be [{D_in}, 2*D_h] (got {tuple(W_in.shape)})")
    D_h = W_in.shape[1] // 2
    device = x_t.device
    if h_prev is not None:
        if not h_prev.is_contiguous():
            raise ValueError("h_prev must be contiguous")
        h_prev = _dev(h_prev, "h_prev", shape=(B, D_h))
    if h_next is None:
        h_next = torch.empty((B, D_h), dtype=torch.float32, device=device)
    else:
        if not h_next.is_contiguous():
            raise ValueError("h_next must be contiguous")
        _dev(h_next, "h_next", shape=(B, D_h))
    if W_out is not None:
        W_out = _dev(W_out, "W_out", ndim=2)
        if W_out.shape[0] != D_h:
            raise ValueError(f"W_out must be [{D_h}, D_out] (got {tuple(W_out.shape)})")
        D_out = W_out.shape[1]
        y_t = torch.empty((B, D_out), dtype=torch.float32, device=device)
    else:
        D_out = D_h
        y_t = None
    nbytes = _lib.mingru_step_workspace_size(B, D_in, D_h, D_out)
    ws = None
    if nbytes:
        ws = _use_workspace(workspace, nbytes, device)
    if decay is None:
        st = _lib.mingru_step(B, D_in, D_h, D_out, _ptr(x_t), _operand(W_in), _operand(W_out),
                              _ptr(h_prev), _ptr(h_next), _ptr(y_t), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(device))
        _check("mingru_step", st)
    else:
        rate, gap, log1p, sat = _decay_args(decay, D_h, (B,), device)
        st = _lib.mingru_step_decayed(B, D_in, D_h, D_out, _ptr(x_t), _operand(W_in), _operand(W_out),
                                      _ptr(rate), _ptr(gap), log1p, _ptr(sat), _ptr(h_prev),
                                      _ptr(h_next), _ptr(y_t), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(device))
        _check("mingru_step_decayed", st)
    return (h_next if y_t is None else y_t), h_next


def minmax_scan(r, s, x0, return_last=False, workspace=None, out=None, out_last=None):
    """MinMax neuron x_{t+1} = max(min(r_t, x_t), s_t) over [B,T,D] inputs.

    Returns x_out [B,T,D] (x_out[:, t] = x_{t+1}), and x_T when ``return_last``.
    """
    r = _dev(r, "r", ndim=3)
    s = _dev(s, "s", shape=r.shape)
    B, T, D = r.shape
    x0 = _dev(x0, "x0", shape=(B, D))
    if out is not None:
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        out = _dev(out, "out", shape=(B, T, D))
    else:
        out = torch.empty_like(r)
    last = None
    if return_last:
        if out_last is not None:
            if not out_last.is_contiguous():
                raise ValueError("out_last must be contiguous")
            last = _dev(out_last, "out_last", shape=(B, D))
        else:
            last = torch.empty((B, D), dtype=torch.float32, device=r.device)
    nbytes = _lib.minmax_scan_workspace_size(B, T, D)
    ws = _use_workspace(workspace, nbytes, r.device)
    st = _lib.minmax_scan(B, T, D, _ptr(r), _ptr(s), _ptr(x0), _ptr(out), _ptr(last), _ptr(ws),
                          ws.numel(), _stream(r.device))
    _check("minmax_scan", st)
    return (out, last) if return_last else out


def minmax_step(r_t, s_t, x_prev, x_next=None):
    """One MinMax token: x_next = max(min(r_t, x_prev), s_t) over [B, D].
    ``x_next`` may be ``x_prev`` (in place)."""
    x_prev = _dev(x_prev, "x_prev", ndim=2)
    if not x_prev.is_contiguous():
        raise ValueError("x_prev must be contiguous")
    B, D = x_prev.shape
    r_t = _dev(r_t, "r_t", shape=(B, D))
    s_t = _dev(s_t, "s_t", shape=(B, D))
    if x_next is None:
        x_next = torch.empty_like(x_prev)
    elif not x_next.is_contiguous():
        raise ValueError("x_next must be contiguous")
    else:
        _dev(x_next, "x_next", shape=(B, D))
    st = _lib.minmax_step(B, D, _ptr(r_t), _ptr(s_t), _ptr(x_prev), _ptr(x_next),
                          _stream(x_prev.device))
    _check("minmax_step", st)
    return x_next


def mingru_scan_backward(k, p, h, dh, h0=None, dh_last=None, workspace=None):
    """Gradients of the scan-only forward (k, p [, h0]) -> h.

    ``h`` is the forward output, ``dh`` [B,T,D] the gradient on it and
    ``dh_last`` [B,D] the gradient on the returned final state.  Returns
    (dk, dp, dh0) in fp32 (dh0 is None when h0 is None)."""
    return _scan_backward(k, p, h, dh, h0, dh_last, workspace, None)


def mingru_scan_backward_decayed(k, p, h, dh, h0=None, dh_last=None, workspace=None, *,
                                 decay_rate, delta_t, log1p_delta=False):
    """``mingru_scan_backward`` of the time-decayed scan (``decay_rate`` [D],
    ``delta_t`` [B,T] as given to ``mingru_forward_decayed``; they get no
    gradient)."""
    return _scan_backward(k, p, h, dh, h0, dh_last, workspace,
                          (decay_rate, delta_t, log1p_delta, None))


def _scan_backward(k, p, h, dh, h0, dh_last, workspace, decay):
    if k.dtype not in (torch.float32, torch.bfloat16) or p.dtype != k.dtype:
        raise TypeError("k and p must both be float32 or both bfloat16")
    if k.dim() != 3 or p.shape != k.shape:
        raise ValueError("k and p must be [B,T,D] of the same shape")
    if k.device.type != "cuda" or p.device != k.device:
        raise ValueError("k and p must be on the same GPU")
    B, T, D = k.shape
    if (k.stride(2) != 1 or p.stride(2) != 1 or k.stride(0) != T * k.stride(1)
            or p.stride(1) != k.stride(1) or p.stride(0) != k.stride(0)):
        k = k.contiguous()
        p = p.contiguous()
    h = _dev(h, "h", shape=(B, T, D))
    dh = _dev(dh, "dh", shape=(B, T, D))
    if h0 is not None:
        h0 = _dev(h0, "h0", shape=(B, D))
    if dh_last is not None:
        dh_last = _dev(dh_last, "dh_last", shape=(B, D))
    dk = torch.empty((B, T, D), dtype=torch.float32, device=k.device)
    dp = torch.empty_like(dk)
    dh0 = torch.empty((B, D), dtype=torch.float32, device=k.device) if h0 is not None else None
    nbytes = _lib.mingru_scan_backward_workspace_size(B, T, D)
    ws = _use_workspace(workspace, nbytes, k.device)
    dtype = SR_BF16 if k.dtype == torch.bfloat16 else SR_F32
    if decay is None:
        st = _lib.mingru_scan_backward(B, T, D, _ptr(k), _ptr(p), k.stride(1), dtype, _ptr(h0),
                                       _ptr(h), _ptr(dh), _ptr(dh_last), _ptr(dk), _ptr(dp),
                                       _ptr(dh0), _ptr(ws), ws.numel(), _stream(k.device))
        _check("mingru_scan_backward", st)
    else:
        rate, gap, log1p, _ = _decay_args(decay, D, (B, T), k.device)
        st = _lib.mingru_scan_backward_decayed(B, T, D, _ptr(k), _ptr(p), k.stride(1), dtype,
                                               _ptr(rate), _ptr(gap), log1p, _ptr(h0), _ptr(h),
                                               _ptr(dh), _ptr(dh_last), _ptr(dk), _ptr(dp),
                                               _ptr(dh0), _ptr(ws), ws.numel(), _stream(k.device))
        _check("mingru_scan_backward_decayed", st)
    return dk, dp, dh0


def minmax_scan_backward(r, s, x0, x_out, dx, dx_last=None, workspace=None):
    """Gradients of the MinMax scan: returns (dr, ds, dx0) in fp32."""
    r = _dev(r, "r", ndim=3)
    B, T, D = r.shape
    s = _dev(s, "s", shape=(B, T, D))
    x0 = _dev(x0, "x0", shape=(B, D))
    x_out = _dev(x_out, "x_out", shape=(B, T, D))
    dx = _dev(dx, "dx", shape=(B, T, D))
    if dx_last is not None:
        dx_last = _dev(dx_last, "dx_last", shape=(B, D))
    dr = torch.empty_like(r)
    ds = torch.empty_like(r)
    dx0 = torch.empty((B, D), dtype=torch.float32, device=r.device)
    nbytes = _lib.minmax_scan_backward_workspace_size(B, T, D)
    ws = _use_workspace(workspace, nbytes, r.device)
    st = _lib.minmax_scan_backward(B, T, D, _ptr(r), _ptr(s), _ptr(x0), _ptr(x_out), _ptr(dx),
                                   _ptr(dx_last), _ptr(dr), _ptr(ds), _ptr(dx0), _ptr(ws),
                                   ws.numel(), _stream(r.device))
    _check("minmax_scan_backward", st)
    return dr, ds, dx0


def set_lookback_spin_limit(polls: int) -> None:
    """Bound on the polls of an unwritten look-back word for scans launched
    afterwards (process-wide; at most LOOKBACK_SPIN_LIMIT, the default).  For
    tests of the timeout path."""
    if not 0 <= polls <= LOOKBACK_SPIN_LIMIT:
        raise ValueError(f"polls must be in [0, {LOOKBACK_SPIN_LIMIT}] (got {polls})")
    _check("scanrnn_set_lookback_spin_limit", _lib.scanrnn_set_lookback_spin_limit(polls))


def workspace_status(ws: torch.Tensor) -> int:
    """Synchronises the current stream and returns the workspace status code."""
    return _lib.scanrnn_workspace_status(_ptr(ws), _stream(ws.device))


class _Scan(torch.autograd.Function):
    """The minGRU scan (k, p [, h0]) -> h, differentiable: the forward is the
    scan-only mingru_forward[_decayed], the backward mingru_scan_backward
    [_decayed] (k, p, h0 get gradients; rates and gaps do not)."""

    @staticmethod
    def forward(ctx, k, p, h0, decay_rate, delta_t, log1p_delta):
        if decay_rate is None:
            h = mingru_forward(k=k, p=p, h0=h0)
        else:
            h = mingru_forward_decayed(k=k, p=p, h0=h0, decay_rate=decay_rate, delta_t=delta_t,
                                       log1p_delta=log1p_delta)
        ctx.save_for_backward(k, p, h0, h, decay_rate, delta_t)
        ctx.log1p_delta = log1p_delta
        return h

    @staticmethod
    def backward(ctx, dh):
        k, p, h0, h, decay_rate, delta_t = ctx.saved_tensors
        dh = dh.contiguous().to(torch.float32)
        if decay_rate is None:
            dk, dp, dh0 = mingru_scan_backward(k, p, h, dh, h0=h0)
        else:
            dk, dp, dh0 = mingru_scan_backward_decayed(k, p, h, dh, h0=h0, decay_rate=decay_rate,
                                                       delta_t=delta_t,
                                                       log1p_delta=ctx.log1p_delta)
        return dk.to(k.dtype), dp.to(p.dtype), dh0, None, None, None


def mingru_scan(k, p, h0=None, *, decay_rate=None, delta_t=None, log1p_delta=False):
    """The minGRU scan k, p [B,T,D] (fp32 or bf16), h0 [B,D] or None -> h
    [B,T,D] fp32, differentiable with respect to k, p and h0 through the
    library's backward kernels (torch autograd only records the call).  With
    ``decay_rate`` [D] and ``delta_t`` [B,T]: the time-decayed scan."""
    if (decay_rate is None) != (delta_t is None):
        raise ValueError("decay_rate and delta_t go together")
    return _Scan.apply(k, p, h0, decay_rate, delta_t, bool(log1p_delta))


class MinGRU:
    """A minGRU layer: W_in [dim, 2*dim*expansion], W_out [dim*expansion, dim].

    ``layer(x)`` with x [B,T,dim] runs the parallel mode and returns y of the
    same shape.  ``layer(x_t, prev_hidden, return_next_prev_hidden=True)`` with
    a single token (x_t [B,dim] or [B,1,dim]) runs one step and returns
    (y_t, h_t); prev_hidden None is the zero state.

    Time decay (the tutorials' decay contract): with ``decay_rate`` (a float
    or a [dim*expansion] tensor of per-channel rates >= 0), a call may pass
    ``delta_t`` -- [B,T] gaps for a sequence, [B] for one token -- and the
    carried state is scaled by exp(-min(rate * gap, 1e4)) before each
    token's write (gap = log1p(delta_t) with ``log1p_delta``).  Without
    ``delta_t`` a call does not decay.  The first call whose rate * gap
    exceeds 1e4 raises one UserWarning per layer (checking synchronises the
    stream; ``warn_saturation=False`` skips the check).
    """

    SATURATION_WARNING = (
        "delta_t gaps exceed the decay clamp (decay_rate * delta_t > 1e4): those tokens "
        "wipe the carried state, and gaps beyond the clamp are no longer told apart; "
        "pass log1p_delta=True or rescale delta_t to keep them distinct")

    def __init__(self, dim: int, expansion: float = 1.0, W_in=None, W_out=None,
                 device="cuda", generator=None, decay_rate=None, log1p_delta=False,
                 warn_saturation=True):
        self.dim = int(dim)
        self.dim_inner = int(dim * expansion)
        if W_in is None:
            W_in = torch.randn(self.dim, 2 * self.dim_inner, generator=generator) / self.dim ** 0.5
        if W_out is None:
            W_out = torch.randn(self.dim_inner, self.dim, generator=generator) / self.dim_inner ** 0.5
        self.W_in = W_in.to(device=device, dtype=torch.float32).contiguous()
        self.W_out = None if W_out is False else W_out.to(device=device, dtype=torch.float32).contiguous()
        self.decay_rate = None
        if decay_rate is not None:
            rate = torch.as_tensor(decay_rate, dtype=torch.float32)
            self.decay_rate = rate.expand(self.dim_inner).to(device).contiguous()
        self.log1p_delta = bool(log1p_delta)
        self.warn_saturation = bool(warn_saturation)
        self._saturated = None
        self._warned = False

    def _decay(self, delta_t):
        if self.decay_rate is None or delta_t is None:
            return None
        if self._saturated is None:
            self._saturated = torch.zeros(1, dtype=torch.int32, device=self.W_in.device)
        return dict(decay_rate=self.decay_rate, delta_t=delta_t.to(torch.float32),
                    log1p_delta=self.log1p_delta, saturated=self._saturated)

    def _maybe_warn(self, dec):
        if dec is None or self._warned or not self.warn_saturation:
            return
        if int(self._saturated.item()) != 0:
            import warnings
            self._warned = True
            warnings.warn(self.SATURATION_WARNING, UserWarning, stacklevel=3)

    def __call__(self, x, prev_hidden=None, return_next_prev_hidden=False, delta_t=None):
        single = x.dim() == 2 or (x.dim() == 3 and x.shape[1] == 1 and prev_hidden is not None)
        dec = self._decay(delta_t)
        if single:
            x_t = x.reshape(x.shape[0], x.shape[-1])
            h = None if prev_hidden is None else prev_hidden.reshape(x_t.shape[0], self.dim_inner)
            if dec is None:
                y_t, h_t = mingru_step(x_t, self.W_in, self.W_out, h)
            else:
                dec["delta_t"] = dec["delta_t"].reshape(x_t.shape[0])
                y_t, h_t = mingru_step_decayed(x_t, self.W_in, self.W_out, h, **dec)
            self._maybe_warn(dec)
            if x.dim() == 3:
                y_t = y_t.unsqueeze(1)
            return (y_t, h_t) if return_next_prev_hidden else y_t
        h0 = None
        if prev_hidden is not None:
            h0 = prev_hidden.reshape(x.shape[0], self.dim_inner)
        if dec is None:
            y, h_last = mingru_forward(x, self.W_in, h0=h0, W_out=self.W_out, return_last=True)
        else:
            y, h_last = mingru_forward_decayed(x, self.W_in, h0=h0, W_out=self.W_out,
                                               return_last=True, **dec)
        self._maybe_warn(dec)
        return (y, h_last) if return_next_prev_hidden else y
