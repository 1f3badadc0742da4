"""RWKV-4 WKV operator for AMD MI355X (gfx950): Python binding of libwkv.

This module only marshals arguments: it checks tensors, takes their device
pointers and the current HIP stream, and calls the C ABI declared in
``include/wkv.h``.  Every step of the computation runs in the HIP kernels of
``libwkv.so``; there is no fallback.  PyTorch provides device memory and
streams.

Operator (aicassindra.com tm_rwkv_math, "The WKV operator: attention with a
fixed decay"), per batch row and channel::

    y_t = (sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u + k_t} v_t)
        / (sum_{i<t} e^{-(t-1-i) w + k_i}     + e^{u + k_t})

with decay rate ``w > 0`` and bonus ``u``; the state (a, b, p) carries the
history with true accumulators e^p a, e^p b (same page, "Numerical
stability: carry the exponent").
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv.so")
ABI_VERSION = 107  # WKV_ABI_VERSION of include/wkv.h that this binding follows

F32 = 0
BF16 = 1
PATH_AUTO = 0
PATH_SERIAL = 1
PATH_CHUNKED = 2
PATH_CHAINED = 3
_PATHS = {"auto": PATH_AUTO, "serial": PATH_SERIAL, "chunked": PATH_CHUNKED,
          "chained": PATH_CHAINED}

_lib = None
_lib_lock = threading.Lock()


class WkvError(RuntimeError):
    """A libwkv call returned a nonzero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libwkv status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libwkv.so with its argument types declared.

    Raises RuntimeError when the library has not been built: there is no
    other implementation to fall back to.
    """
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950) before using linear_attention_rnn_forward_amd")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.wkv_forward_workspace_size.restype = sz
        L.wkv_forward_workspace_size.argtypes = [i64, i64, i64, i32]
        L.wkv_forward_workspace_size_path.restype = sz
        L.wkv_forward_workspace_size_path.argtypes = [i64, i64, i64, i32, i32]
        L.wkv_forward.restype = i32
        L.wkv_forward.argtypes = [i64, i64, i64, i32] + [vp] * 11 + [vp, sz, vp]
        L.wkv_forward_path.restype = i32
        L.wkv_forward_path.argtypes = [i64, i64, i64, i32, i32] + [vp] * 11 + [vp, sz, vp]
        L.wkv_forward_gated.restype = i32
        L.wkv_forward_gated.argtypes = [i64, i64, i64, i32, i32] + [vp] * 12 + [vp, sz, vp]
        L.wkv_step.restype = i32
        L.wkv_step.argtypes = [i64, i64, i64, i32] + [vp] * 11 + [vp]
        L.wkv_step_gated.restype = i32
        L.wkv_step_gated.argtypes = [i64, i64, i64, i32] + [vp] * 12 + [vp]
        L.wkv_session_bytes.restype = sz
        L.wkv_session_bytes.argtypes = [i64, i64, i32, i32]
        L.wkv_session_save.restype = i32
        L.wkv_session_save.argtypes = [i64, i64, i64, i32, i64, vp, vp, vp, vp, i32, vp, sz, vp]
        L.wkv_session_load.restype = i32
        L.wkv_session_load.argtypes = [i64, i64, i64, i32, i64, vp, sz, vp, vp, vp, vp, i32, vp]
        L.wkv_backward_workspace_size.restype = sz
        L.wkv_backward_workspace_size.argtypes = [i64, i64, i64]
        L.wkv_backward.restype = i32
        L.wkv_backward.argtypes = [i64, i64, i64, i32] + [vp] * 9 + [vp, sz, vp]
        L.wkv_saved_states_bytes.restype = sz
        L.wkv_saved_states_bytes.argtypes = [i64, i64, i64]
        L.wkv_forward_save.restype = i32
        L.wkv_forward_save.argtypes = [i64, i64, i64, i32] + [vp] * 6 + [vp]
        L.wkv_backward_saved_workspace_size.restype = sz
        L.wkv_backward_saved_workspace_size.argtypes = [i64, i64]
        L.wkv_backward_saved.restype = i32
        L.wkv_backward_saved.argtypes = [i64, i64, i64, i32] + [vp] * 10 + [vp, sz, vp]
        L.wkv_token_shift.restype = i32
        L.wkv_token_shift.argtypes = [i64, i64, i64, i32] + [vp] * 9 + [vp]
        L.wkv_status_string.restype = ctypes.c_char_p
        L.wkv_mat_forward.restype = i32
        L.wkv_mat_forward.argtypes = [i64, i64, i64, i32] + [vp] * 4 + [i32] + [vp] * 4
        L.wkv_mat_forward_path.restype = i32
        L.wkv_mat_forward_path.argtypes = [i64, i64, i64, i32, i32] + [vp] * 4 + [i32] + [vp] * 4
        L.wkv_mat_step.restype = i32
        L.wkv_mat_step.argtypes = [i64, i64, i64, i32] + [vp] * 4 + [i32] + [vp] * 4
        L.wkv_status_string.argtypes = [i32]
        L.wkv_last_error.restype = ctypes.c_char_p
        L.wkv_last_error.argtypes = []
        L.wkv_abi_version.restype = i32
        L.wkv_abi_version.argtypes = []
        L.wkv_forward_noalloc.restype = i32
        L.wkv_forward_noalloc.argtypes = [i64, i64, i64, i32] + [vp] * 11 + [vp]
        L.wkv_forward_auto_path.restype = i32
        L.wkv_forward_auto_path.argtypes = [i64, i64, i64, i32]
        L.wkv_bounded_wait_failures.restype = i32
        L.wkv_bounded_wait_failures.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        got = int(L.wkv_abi_version())
        if got != ABI_VERSION:
            # buffer sizes and layouts (the saved states among them) differ
            # between versions: refuse rather than pass mis-sized buffers
            raise RuntimeError(f"{LIB_PATH} has ABI version {got}, this binding needs {ABI_VERSION}: "
                               "rebuild it with __graft_entry__.build()")
        _lib = L
    return _lib


def auto_path(B: int, T: int, C: int, dtype: int = F32) -> str:
    """The execution path wkv_forward takes for these sizes on the current device."""
    code = lib().wkv_forward_auto_path(B, T, C, dtype)
    check(min(code, 0))
    return {v: k for k, v in _PATHS.items()}[code]


def bounded_wait_failures() -> int:
    """Bounded waits (chunked look-back, matrix ring) that gave up on the
    current device since the library was loaded; synchronous."""
    n = ctypes.c_uint64(0)
    check(lib().wkv_bounded_wait_failures(ctypes.byref(n)))
    return int(n.value)


def check(status: int) -> None:
    """Raise WkvError for a nonzero libwkv status."""
    if status != 0:
        L = lib()
        msg = L.wkv_last_error().decode() or L.wkv_status_string(status).decode()
        raise WkvError(status, msg)


# ---------------------------------------------------------------------------
# tensor helpers (torch is imported lazily: the C ABI itself never sees it)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"k, v must be float32 or bfloat16, got {t.dtype}")


def _need(t, name, shape=None, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


_workspaces: dict = {}


def _workspace(device, nbytes: int):
    """A cached device workspace of at least nbytes for `device` (contents are
    irrelevant to the library).  Reused across calls on the same stream."""
    if nbytes == 0:
        return None
    torch = _torch()
    key = (device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_size(B: int, T: int, C: int, dtype: int = F32, path: str = "auto") -> int:
    """Bytes of workspace wkv_forward needs for these sizes on the current device."""
    return int(lib().wkv_forward_workspace_size_path(B, T, C, dtype, _PATHS[path]))


# ---------------------------------------------------------------------------
# public calls
# ---------------------------------------------------------------------------

def forward(k, v, w, u, state=None, return_state=False, path="auto", out=None, state_out=None,
            workspace=None, r=None):
    """Training / prefill form over all positions.

    k, v: [B,T,C] float32 or bfloat16 (same dtype); w, u: [C] float32.
    state: None (empty history) or (a, b, p), each [B,C] float32.
    r: None, or the receptance [B,T,C] (dtype of k): the output is then
    sigmoid(r) * wkv (the gate fused into the same pass).
    Returns y [B,T,C] (dtype of k), or (y, (a, b, p)) with return_state.
    path: "auto", or "serial", "chained", "chunked" to force an execution path.
    """
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3:
        raise ValueError("k must be [B,T,C]")
    B, T, C = k.shape
    dev = k.device
    dt = _dtype_code(k)
    _need(v, "v", k.shape, k.dtype, dev)
    _need(w, "w", (C,), torch.float32, dev)
    _need(u, "u", (C,), torch.float32, dev)
    a_in = b_in = p_in = None
    if state is not None:
        a_in, b_in, p_in = (_need(x, n, (B, C), torch.float32, dev)
                            for x, n in zip(state, ("a_in", "b_in", "p_in")))
    y = out if out is not None else torch.empty_like(k)
    _need(y, "out", k.shape, k.dtype, dev)
    a_out = b_out = p_out = None
    if return_state or state_out is not None:
        if state_out is None:
            state_out = tuple(torch.empty((B, C), dtype=torch.float32, device=dev) for _ in range(3))
        a_out, b_out, p_out = (_need(x, n, (B, C), torch.float32, dev)
                               for x, n in zip(state_out, ("a_out", "b_out", "p_out")))
    if r is not None:
        _need(r, "r", k.shape, k.dtype, dev)
    code = _PATHS[path]
    need = int(lib().wkv_forward_workspace_size_path(B, T, C, dt, code))
    ws = workspace if workspace is not None else _workspace(dev, need)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    with torch.cuda.device(dev):
        if r is None:
            check(lib().wkv_forward_path(B, T, C, dt, code, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                         _ptr(y), _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(a_out),
                                         _ptr(b_out), _ptr(p_out), _ptr(ws), ws_bytes, _stream(dev)))
        else:
            check(lib().wkv_forward_gated(B, T, C, dt, code, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                          _ptr(r), _ptr(y), _ptr(a_in), _ptr(b_in), _ptr(p_in),
                                          _ptr(a_out), _ptr(b_out), _ptr(p_out), _ptr(ws), ws_bytes,
                                          _stream(dev)))
    if return_state or state_out is not None:
        return y, (a_out, b_out, p_out)
    return y


def forward_noalloc(k, v, w, u, out, state=None, state_out=None):
    """wkv_forward without a workspace and without allocating anything: the
    chunked path uses the library's fixed device array (wkv_forward_noalloc).
    The caller passes every output: out [B,T,C] (dtype of k) and, if the
    final state is wanted, state_out = (a, b, p) [B,C] float32.  Returns out."""
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3:
        raise ValueError("k must be [B,T,C]")
    B, T, C = k.shape
    dev = k.device
    dt = _dtype_code(k)
    _need(v, "v", k.shape, k.dtype, dev)
    _need(w, "w", (C,), torch.float32, dev)
    _need(u, "u", (C,), torch.float32, dev)
    _need(out, "out", k.shape, k.dtype, dev)
    a_in = b_in = p_in = a_out = b_out = p_out = None
    if state is not None:
        a_in, b_in, p_in = (_need(x, n, (B, C), torch.float32, dev)
                            for x, n in zip(state, ("a_in", "b_in", "p_in")))
    if state_out is not None:
        a_out, b_out, p_out = (_need(x, n, (B, C), torch.float32, dev)
                               for x, n in zip(state_out, ("a_out", "b_out", "p_out")))
    with torch.cuda.device(dev):
        check(lib().wkv_forward_noalloc(B, T, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(a_out),
                                        _ptr(b_out), _ptr(p_out), _stream(dev)))
    return out


def backward_workspace_size(B: int, T: int, C: int) -> int:
    """Bytes of workspace wkv_backward needs for these sizes."""
    return int(lib().wkv_backward_workspace_size(B, T, C))


SAVED_STATE_TOKENS = 16


def saved_states_shape(B: int, T: int, C: int):
    """Shape of forward_save's states: [B, ceil(T/16), 2, C] float32 (r, q per
    channel: the history sums are r e^q and e^q)."""
    return (B, (T + SAVED_STATE_TOKENS - 1) // SAVED_STATE_TOKENS, 2, C)


def forward_save(k, v, w, u, out=None, states=None):
    """forward(k, v, w, u) from the empty history that also saves the state
    before every 16-token sub-chunk (wkv_forward_save), for backward(...,
    states=...).  Returns (y, states); states is [B, ceil(T/16), 2, C]
    float32."""
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3:
        raise ValueError("k must be [B,T,C]")
    B, T, C = k.shape
    dev = k.device
    dt = _dtype_code(k)
    _need(v, "v", k.shape, k.dtype, dev)
    _need(w, "w", (C,), torch.float32, dev)
    _need(u, "u", (C,), torch.float32, dev)
    y = out if out is not None else torch.empty_like(k)
    _need(y, "out", k.shape, k.dtype, dev)
    shape = saved_states_shape(B, T, C)
    if states is None:
        states = torch.empty(shape, dtype=torch.float32, device=dev)
    _need(states, "states", shape, torch.float32, dev)
    with torch.cuda.device(dev):
        check(lib().wkv_forward_save(B, T, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                     _ptr(states), _stream(dev)))
    return y, states


def backward(k, v, w, u, gy, out=None, workspace=None, states=None):
    """Gradients of sum(gy * forward(k, v, w, u)) from the empty history.

    k, v, gy: [B,T,C] float32 or bfloat16 (same dtype); w, u: [C] float32.
    Returns (gk, gv, gw, gu): gk, gv [B,T,C] in the dtype of k, gw, gu [C]
    float32 (summed over batch and tokens).  out: optional preallocated
    (gk, gv, gw, gu).  states: the states forward_save saved for the same
    inputs (wkv_backward_saved: k, v are then read once less), or None.
    """
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3:
        raise ValueError("k must be [B,T,C]")
    B, T, C = k.shape
    dev = k.device
    dt = _dtype_code(k)
    _need(v, "v", k.shape, k.dtype, dev)
    _need(gy, "gy", k.shape, k.dtype, dev)
    _need(w, "w", (C,), torch.float32, dev)
    _need(u, "u", (C,), torch.float32, dev)
    if out is None:
        out = (torch.empty_like(k), torch.empty_like(k),
               torch.empty(C, dtype=torch.float32, device=dev),
               torch.empty(C, dtype=torch.float32, device=dev))
    gk, gv, gw, gu = out
    _need(gk, "gk", k.shape, k.dtype, dev)
    _need(gv, "gv", k.shape, k.dtype, dev)
    _need(gw, "gw", (C,), torch.float32, dev)
    _need(gu, "gu", (C,), torch.float32, dev)
    if states is not None:
        _need(states, "states", saved_states_shape(B, T, C), torch.float32, dev)
        need = int(lib().wkv_backward_saved_workspace_size(B, C))
    else:
        need = int(lib().wkv_backward_workspace_size(B, T, C))
    ws = workspace if workspace is not None else _workspace(dev, need)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    with torch.cuda.device(dev):
        if states is not None:
            check(lib().wkv_backward_saved(B, T, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                           _ptr(gy), _ptr(states), _ptr(gk), _ptr(gv), _ptr(gw),
                                           _ptr(gu), _ptr(ws), ws_bytes, _stream(dev)))
        else:
            check(lib().wkv_backward(B, T, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(gy),
                                     _ptr(gk), _ptr(gv), _ptr(gw), _ptr(gu), _ptr(ws), ws_bytes,
                                     _stream(dev)))
    return gk, gv, gw, gu


def backward_saved_workspace_size(B: int, C: int) -> int:
    """Bytes of workspace wkv_backward_saved needs."""
    return int(lib().wkv_backward_saved_workspace_size(B, C))


def step(state, k, v, w, u, out=None, state_out=None, inplace=False, r=None):
    """One decode token for every (layer, sequence, channel).

    state: (a, b, p), each [L,S,C] float32 (p = -inf for an empty history).
    k, v: [L,S,C] float32 or bfloat16; w, u: [L,C] float32.
    r: None, or the receptance [L,S,C] (dtype of k): y = sigmoid(r) * wkv.
    Returns (y, (a', b', p')).  inplace=True writes the new state into `state`.
    """
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3:
        raise ValueError("k must be [L,S,C]")
    Ln, S, C = k.shape
    dev = k.device
    dt = _dtype_code(k)
    _need(v, "v", k.shape, k.dtype, dev)
    _need(w, "w", (Ln, C), torch.float32, dev)
    _need(u, "u", (Ln, C), torch.float32, dev)
    a_in, b_in, p_in = (_need(x, n, (Ln, S, C), torch.float32, dev)
                        for x, n in zip(state, ("a", "b", "p")))
    if inplace:
        state_out = (a_in, b_in, p_in)
    elif state_out is None:
        state_out = tuple(torch.empty_like(a_in) for _ in range(3))
    a_out, b_out, p_out = (_need(x, n, (Ln, S, C), torch.float32, dev)
                           for x, n in zip(state_out, ("a_out", "b_out", "p_out")))
    y = out if out is not None else torch.empty_like(k)
    _need(y, "out", k.shape, k.dtype, dev)
    if r is not None:
        _need(r, "r", k.shape, k.dtype, dev)
    with torch.cuda.device(dev):
        if r is None:
            check(lib().wkv_step(Ln, S, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                 _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(a_out), _ptr(b_out),
                                 _ptr(p_out), _stream(dev)))
        else:
            check(lib().wkv_step_gated(Ln, S, C, dt, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                       _ptr(y), _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(a_out),
                                       _ptr(b_out), _ptr(p_out), _stream(dev)))
    return y, (a_out, b_out, p_out)


def token_shift(x, mu_r, mu_k, mu_v, x_prev=None, return_last=False, out=None):
    """Two-tap causal lerp for the three blends; x [B,T,C] float32/bfloat16,
    mu_* [C] float32, x_prev [B,C] (dtype of x) or None (zeros).
    out: None, or (xr, xk, xv) preallocated like x.
    Returns (xr, xk, xv) or (xr, xk, xv, x_last)."""
    torch = _torch()
    _need(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B,T,C]")
    B, T, C = x.shape
    dev = x.device
    dt = _dtype_code(x)
    for m, n in ((mu_r, "mu_r"), (mu_k, "mu_k"), (mu_v, "mu_v")):
        _need(m, n, (C,), torch.float32, dev)
    if x_prev is not None:
        _need(x_prev, "x_prev", (B, C), x.dtype, dev)
    if out is None:
        xr, xk, xv = (torch.empty_like(x) for _ in range(3))
    else:
        xr, xk, xv = (_need(t, n, x.shape, x.dtype, dev) for t, n in zip(out, ("xr", "xk", "xv")))
    x_last = torch.empty((B, C), dtype=x.dtype, device=dev) if return_last else None
    with torch.cuda.device(dev):
        check(lib().wkv_token_shift(B, T, C, dt, _ptr(x), _ptr(x_prev), _ptr(mu_r), _ptr(mu_k),
                                    _ptr(mu_v), _ptr(xr), _ptr(xk), _ptr(xv), _ptr(x_last),
                                    _stream(dev)))
    if return_last:
        return xr, xk, xv, x_last
    return xr, xk, xv


# ---------------------------------------------------------------------------
# session save / resume
# ---------------------------------------------------------------------------

def _ptr_array(ts):
    arr = (ctypes.c_void_p * max(len(ts), 1))(*[t.data_ptr() for t in ts])
    return arr if ts else None


def session_bytes(L: int, C: int, dtype: int = F32, n_shift: int = 0) -> int:
    """Bytes of one sequence's session blob (header, a, b, p, shifted tokens)."""
    return int(lib().wkv_session_bytes(L, C, dtype, n_shift))


def save_session(state, seq, shifts=()):
    """The state of sequence `seq` of a decode batch as bytes.

    state: (a, b, p), each [L,S,C] float32 on the GPU; shifts: shifted-token
    arrays [L,S,C] (float32 or bfloat16, all one dtype).  Copies into pinned
    host memory on the current stream and waits for them."""
    torch = _torch()
    a, b, p = state
    _need(a, "a")
    Ln, S, C = a.shape
    dev = a.device
    for x, n in zip(state, ("a", "b", "p")):
        _need(x, n, (Ln, S, C), torch.float32, dev)
    dt = _dtype_code(shifts[0]) if shifts else F32
    for i, x in enumerate(shifts):
        _need(x, f"shifts[{i}]", (Ln, S, C), shifts[0].dtype, dev)
    n = session_bytes(Ln, C, dt, len(shifts))
    if n == 0:
        raise ValueError("invalid session shape")
    blob = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    with torch.cuda.device(dev):
        check(lib().wkv_session_save(Ln, S, C, dt, seq, _ptr(a), _ptr(b), _ptr(p),
                                     _ptr_array(list(shifts)), len(shifts), _ptr(blob), n,
                                     _stream(dev)))
        torch.cuda.current_stream(dev).synchronize()
    return bytes(blob.numpy())


def load_session(blob, state, seq, shifts=()):
    """Write a blob from save_session into sequence `seq` of `state` (and of
    `shifts`), on the current stream; waits for the copies."""
    torch = _torch()
    a, b, p = state
    _need(a, "a")
    Ln, S, C = a.shape
    dev = a.device
    for x, n in zip(state, ("a", "b", "p")):
        _need(x, n, (Ln, S, C), torch.float32, dev)
    dt = _dtype_code(shifts[0]) if shifts else F32
    for i, x in enumerate(shifts):
        _need(x, f"shifts[{i}]", (Ln, S, C), shifts[0].dtype, dev)
    host = torch.frombuffer(bytearray(blob), dtype=torch.uint8).pin_memory()
    with torch.cuda.device(dev):
        check(lib().wkv_session_load(Ln, S, C, dt, seq, _ptr(host), host.numel(), _ptr(a), _ptr(b),
                                     _ptr(p), _ptr_array(list(shifts)), len(shifts), _stream(dev)))
        torch.cuda.current_stream(dev).synchronize()


# ---------------------------------------------------------------------------
# matrix-valued state (RWKV-5 Eagle / RWKV-6 Finch)
# ---------------------------------------------------------------------------

MAT_HEAD_DIM = 64
MAT_DECAY_PER_CHANNEL = 0
MAT_DECAY_PER_TOKEN = 1
_MAT_PATHS = {"auto": 0, "chunked": 1, "tokenwise": 2}


def _mat_z(z, shape_token, shape_channel, dtype, dev):
    torch = _torch()
    if tuple(z.shape) == tuple(shape_token):
        _need(z, "z", shape_token, dtype, dev)
        return MAT_DECAY_PER_TOKEN
    _need(z, "z", shape_channel, torch.float32, dev)
    return MAT_DECAY_PER_CHANNEL


def mat_forward(r, k, v, z, state=None, return_state=False, path="auto", out=None,
                state_out=None):
    """S_t = diag(d_t) S_{t-1} + k_t v_t^T, y_t = r_t^T S_t, d_t = exp(-softplus(z_t)),
    per batch row and head of 64 channels (vanos001.github.io "RWKV (Attention-RNN
    Hybrid)", the versions table and the matrix-form recurrence under it).

    r, k, v: [B,T,C] float32 or bfloat16, C = 64 H.  z: [B,T,C] like r (Finch,
    per-token decay) or [C] float32 (Eagle, per-channel decay).  state: None
    (zero) or [B,H,64,64] float32.  path: "auto", "chunked" (bf16 only) or
    "tokenwise".  Returns y, or (y, S_T) with return_state.
    """
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3 or k.shape[2] % MAT_HEAD_DIM != 0:
        raise ValueError("k must be [B,T,C] with C a multiple of 64")
    B, T, C = k.shape
    H = C // MAT_HEAD_DIM
    dev = k.device
    dt = _dtype_code(k)
    _need(r, "r", k.shape, k.dtype, dev)
    _need(v, "v", k.shape, k.dtype, dev)
    z_mode = _mat_z(z, k.shape, (C,), k.dtype, dev)
    st_shape = (B, H, MAT_HEAD_DIM, MAT_HEAD_DIM)
    if state is not None:
        _need(state, "state", st_shape, torch.float32, dev)
    if return_state and state_out is None:
        state_out = torch.empty(st_shape, dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", st_shape, torch.float32, dev)
    y = out if out is not None else torch.empty_like(k)
    _need(y, "out", k.shape, k.dtype, dev)
    with torch.cuda.device(dev):
        check(lib().wkv_mat_forward_path(B, T, H, dt, _MAT_PATHS[path], _ptr(r), _ptr(k), _ptr(v),
                                         _ptr(z), z_mode, _ptr(state), _ptr(state_out), _ptr(y),
                                         _stream(dev)))
    return (y, state_out) if return_state else y


def mat_step(state, r, k, v, z, out=None, state_out=None, inplace=False):
    """One decode token for every (layer, sequence) row and head.

    state: [L,S,H,64,64] float32.  r, k, v: [L,S,C] float32 or bfloat16.
    z: [L,S,C] like r (per token) or [L,C] float32 (per channel).
    Returns (y, S').  inplace=True writes S' into `state`.
    """
    torch = _torch()
    _need(k, "k")
    if k.dim() != 3 or k.shape[2] % MAT_HEAD_DIM != 0:
        raise ValueError("k must be [L,S,C] with C a multiple of 64")
    Ln, S, C = k.shape
    H = C // MAT_HEAD_DIM
    dev = k.device
    dt = _dtype_code(k)
    _need(r, "r", k.shape, k.dtype, dev)
    _need(v, "v", k.shape, k.dtype, dev)
    z_mode = _mat_z(z, k.shape, (Ln, C), k.dtype, dev)
    st_shape = (Ln, S, H, MAT_HEAD_DIM, MAT_HEAD_DIM)
    _need(state, "state", st_shape, torch.float32, dev)
    if inplace:
        state_out = state
    elif state_out is None:
        state_out = torch.empty_like(state)
    _need(state_out, "state_out", st_shape, torch.float32, dev)
    y = out if out is not None else torch.empty_like(k)
    _need(y, "out", k.shape, k.dtype, dev)
    with torch.cuda.device(dev):
        check(lib().wkv_mat_step(Ln, S, H, dt, _ptr(r), _ptr(k), _ptr(v), _ptr(z), z_mode,
                                 _ptr(state), _ptr(state_out), _ptr(y), _stream(dev)))
    return y, state_out
