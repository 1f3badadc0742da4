"""CPU fp64 oracle for the RWKV-4 WKV operator.

TEST INFRASTRUCTURE ONLY.  This package checks the HIP library; it is not
part of it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
here.  It shares no code with ``linear_attention_rnn_forward_amd`` and never
imports it.

What each routine follows (pages cited by address and section):

* ``forward`` / ``step`` — the max-stabilised (a, b, p) recurrence:
  aiwiki.thehackersbrain.dev/entries/rwkv, the ``wkv_step`` listing, and
  aicassindra.com tm_rwkv_math, "Numerical stability: carry the exponent".
  Implemented in C (``wkv_oracle.c``), fp64.
* ``direct`` — the summed definition of wkv_t, O(T^2) (tm_rwkv_math, "The
  WKV operator: attention with a fixed decay"), in C, fp64.
* ``direct_np`` — the same definition written a second, independent way in
  NumPy (a causal weight matrix, normalised row by row).
* ``naive`` — the unstabilised two-accumulator recurrence (tm_rwkv_math,
  "Why it collapses into a recurrence") evaluated in a chosen NumPy float
  type; used only to show the overflow the stabilised form avoids.
* ``token_shift`` — the two-tap causal lerp (tm_rwkv_math, "Token shift: a
  two-tap causal convolution"), in C, fp64.
* ``backward`` — the gradients of the summed definition of wkv_t (empty
  history) with respect to k, v, w and u, written out in NumPy fp64 from
  the softmax form of "The WKV operator" (tm_rwkv_math): every output is a
  weighted mean of values, so d wkv_t / d(term exponent) = weight * (v_i -
  wkv_t).  O(T^2) per column.
* ``sigmoid`` / ``gate`` / ``forward_gated`` / ``step_gated`` — the
  receptance gate o = sigmoid(r) * wkv applied elementwise to the output of
  ``forward`` / ``step`` (tm_rwkv_math, "Receptance: the gate on the way
  out"), NumPy fp64.  The state is the plain recurrence's.

The matrix-valued-state operator of RWKV-5/6 (Eagle, Finch) has its own
NumPy fp64 module, ``oracle.matrix_state``, pinned by
``tests/test_oracle_matrix_pins.py``.

Pins (what ties these to the pages rather than to themselves) live in
``tests/test_oracle_pins.py``.  Inputs are promoted exactly to fp64 from
whatever they are stored as (fp32, or bf16 widened to fp32), so the oracle
sees the values the GPU sees.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _bind(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    for name in ("wkv_oracle_forward", "wkv_oracle_step", "wkv_oracle_direct"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64] + [dp] * 11
    lib.wkv_oracle_token_shift.restype = ctypes.c_int
    lib.wkv_oracle_token_shift.argtypes = [i64, i64, i64] + [dp] * 9
    lib.wkv_oracle_threads.restype = ctypes.c_int
    lib.wkv_oracle_threads.argtypes = []
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _bind(_build.LIB)
    return _LIB


@contextlib.contextmanager
def library(path: str):
    """Temporarily route every call to another build of wkv_oracle.c (used by
    the test that plants mistakes in copies of the oracle)."""
    global _LIB
    saved = _LIB
    _LIB = _bind(path)
    try:
        yield
    finally:
        _LIB = saved


def threads() -> int:
    """OpenMP threads the C oracle runs with."""
    return int(_lib().wkv_oracle_threads())


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _state_in(state, n_shape):
    if state is None:
        return None, None, None
    a, b, p = (_f64(s).reshape(n_shape) for s in state)
    return a, b, p


def forward(k, v, w, u, state=None):
    """Stabilised recurrence over [B,T,C]; returns (y, (a, b, p)) in fp64.

    ``state`` is None (empty history) or a triple of [B,C] arrays.
    """
    k = _f64(k)
    v = _f64(v)
    B, T, C = k.shape
    assert v.shape == k.shape
    w = _f64(w).reshape(C)
    u = _f64(u).reshape(C)
    a_in, b_in, p_in = _state_in(state, (B, C))
    y = np.empty_like(k)
    a_out = np.empty((B, C))
    b_out = np.empty((B, C))
    p_out = np.empty((B, C))
    rc = _lib().wkv_oracle_forward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                   _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(y),
                                   _ptr(a_out), _ptr(b_out), _ptr(p_out))
    assert rc == 0
    return y, (a_out, b_out, p_out)


def direct(k, v, w, u, state=None):
    """Summed definition, O(T^2) per column; returns (y, (a, b, p)) in fp64."""
    k = _f64(k)
    v = _f64(v)
    B, T, C = k.shape
    w = _f64(w).reshape(C)
    u = _f64(u).reshape(C)
    a_in, b_in, p_in = _state_in(state, (B, C))
    y = np.empty_like(k)
    a_out = np.empty((B, C))
    b_out = np.empty((B, C))
    p_out = np.empty((B, C))
    rc = _lib().wkv_oracle_direct(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                  _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(y),
                                  _ptr(a_out), _ptr(b_out), _ptr(p_out))
    assert rc == 0
    return y, (a_out, b_out, p_out)


def step(state, k, v, w, u):
    """One decode step over [L,S,C] with per-layer w,u [L,C].

    Returns (y, (a, b, p)), all [L,S,C] fp64.
    """
    k = _f64(k)
    v = _f64(v)
    L, S, C = k.shape
    w = _f64(w).reshape(L, C)
    u = _f64(u).reshape(L, C)
    a_in, b_in, p_in = _state_in(state, (L, S, C))
    y = np.empty_like(k)
    a_out = np.empty((L, S, C))
    b_out = np.empty((L, S, C))
    p_out = np.empty((L, S, C))
    rc = _lib().wkv_oracle_step(L, S, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v),
                                _ptr(a_in), _ptr(b_in), _ptr(p_in), _ptr(y),
                                _ptr(a_out), _ptr(b_out), _ptr(p_out))
    assert rc == 0
    return y, (a_out, b_out, p_out)


def token_shift(x, mu_r, mu_k, mu_v, x_prev=None):
    """Two-tap causal lerp over [B,T,C]; returns (xr, xk, xv, x_last)."""
    x = _f64(x)
    B, T, C = x.shape
    mu_r, mu_k, mu_v = (_f64(m).reshape(C) for m in (mu_r, mu_k, mu_v))
    xp = None if x_prev is None else _f64(x_prev).reshape(B, C)
    xr = np.empty_like(x)
    xk = np.empty_like(x)
    xv = np.empty_like(x)
    x_last = np.empty((B, C))
    rc = _lib().wkv_oracle_token_shift(B, T, C, _ptr(x), _ptr(xp), _ptr(mu_r), _ptr(mu_k),
                                       _ptr(mu_v), _ptr(xr), _ptr(xk), _ptr(xv), _ptr(x_last))
    assert rc == 0
    return xr, xk, xv, x_last


def direct_np(k, v, w, u):
    """Summed definition written independently of the C code (empty history).

    For each column, row t of a [T,T] matrix holds the exponent of every term
    of wkv_t: -(t-1-i) w + k_i for i < t, u + k_t on the diagonal, and -inf
    above it (tm_rwkv_math, "The WKV operator").  Each row is normalised after
    subtracting its maximum; wkv_t is that row's weights applied to v.
    Only for small T: it materialises B*C*T*T doubles.
    """
    k = _f64(k)
    v = _f64(v)
    B, T, C = k.shape
    w = _f64(w).reshape(C)
    u = _f64(u).reshape(C)
    t_idx = np.arange(T)[:, None]
    i_idx = np.arange(T)[None, :]
    dist = (t_idx - 1 - i_idx).astype(np.float64)          # t-1-i
    past = i_idx < t_idx
    now = i_idx == t_idx
    y = np.empty_like(k)
    for bb in range(B):
        for c in range(C):
            kc = k[bb, :, c]
            X = np.full((T, T), -np.inf)
            X[past] = (-dist * w[c] + kc[None, :])[past]
            X[now] = u[c] + kc
            X = X - X.max(axis=1, keepdims=True)
            W = np.exp(X)
            y[bb, :, c] = (W @ v[bb, :, c]) / W.sum(axis=1)
    return y


def naive(k, v, w, u, dtype=np.float64):
    """Unstabilised recurrence in ``dtype`` (tm_rwkv_math, "Why it collapses
    into a recurrence"):

        wkv_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t})
        a_t   = e^{-w} a_{t-1} + e^{k_t} v_t,   b_t = e^{-w} b_{t-1} + e^{k_t}
        a_0 = b_0 = 0

    Every operation is carried out in ``dtype`` (NumPy rounds each float16 /
    float32 operation to that type).  Returns (y, a_hist, b_hist) with a_hist[t]
    and b_hist[t] the accumulators after token t.  Overflow is the point, so
    floating-point warnings are silenced.
    """
    dt = np.dtype(dtype)
    k = np.asarray(k, dtype=dt)
    v = np.asarray(v, dtype=dt)
    B, T, C = k.shape
    w = np.asarray(w, dtype=dt).reshape(C)
    u = np.asarray(u, dtype=dt).reshape(C)
    y = np.empty((B, T, C), dtype=dt)
    a_hist = np.empty((B, T, C), dtype=dt)
    b_hist = np.empty((B, T, C), dtype=dt)
    with np.errstate(all="ignore"):
        decay = np.exp(-w)
        a = np.zeros((B, C), dtype=dt)
        b = np.zeros((B, C), dtype=dt)
        for t in range(T):
            kt = k[:, t, :]
            vt = v[:, t, :]
            e_now = np.exp(u + kt)
            y[:, t, :] = (a + e_now * vt) / (b + e_now)
            ek = np.exp(kt)
            a = decay * a + ek * vt
            b = decay * b + ek
            a_hist[:, t, :] = a
            b_hist[:, t, :] = b
    return y, a_hist, b_hist


def sigmoid(r):
    """The logistic function 1 / (1 + e^{-r}) in fp64 (tm_rwkv_math,
    "Receptance: the gate on the way out"), written in the form that does not
    overflow: e^{r} / (1 + e^{r}) for r < 0."""
    r = _f64(r)
    e = np.exp(-np.abs(r))
    return np.where(r >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate(y, r):
    """o = sigmoid(r) * y, elementwise (the receptance gate)."""
    return sigmoid(r) * _f64(y)


def forward_gated(k, v, r, w, u, state=None):
    """``forward`` followed by the receptance gate: (o, state)."""
    y, st = forward(k, v, w, u, state=state)
    return gate(y, r), st


def step_gated(state, k, v, r, w, u):
    """``step`` followed by the receptance gate: (o, state')."""
    y, st = step(state, k, v, w, u)
    return gate(y, r), st


def backward(k, v, w, u, gy, magnitude=False):
    """Gradients of L = sum(gy * wkv) for wkv over [B,T,C] from the empty
    history: returns (gk, gv [B,T,C], gw, gu [C]) in fp64.

    magnitude=True returns instead the same sums with every term made
    non-negative -- gy_t alpha[t,i] by its absolute value and (v_i - wkv_t)
    by |v_i| + |wkv_t| -- the scale against which the rounding error of any
    evaluation order of those sums is measured.

    For one column, wkv_t = sum_i alpha[t,i] v_i with alpha row t the softmax
    of the exponents X[t,i] = -(t-1-i) w + k_i (i < t) and u + k_t (i = t)
    (tm_rwkv_math, "The WKV operator: attention with a fixed decay").  Then
    d wkv_t / d v_i = alpha[t,i] and d wkv_t / d X[t,i] = alpha[t,i] (v_i -
    wkv_t); X[t,i] moves one for one with k_i, with u on the diagonal, and by
    -(t-1-i) with w.  Only for small T (materialises T x T per column).
    """
    k = _f64(k)
    v = _f64(v)
    g = _f64(gy)
    B, T, C = k.shape
    w = _f64(w).reshape(C)
    u = _f64(u).reshape(C)
    t_idx = np.arange(T)[:, None]
    i_idx = np.arange(T)[None, :]
    dist = (t_idx - 1 - i_idx).astype(np.float64)
    past = i_idx < t_idx
    now = i_idx == t_idx
    gk = np.zeros_like(k)
    gv = np.zeros_like(k)
    gw = np.zeros(C)
    gu = np.zeros(C)
    for bb in range(B):
        for c in range(C):
            kc, vc, gc = k[bb, :, c], v[bb, :, c], g[bb, :, c]
            X = np.full((T, T), -np.inf)
            X[past] = (-dist * w[c] + kc[None, :])[past]
            X[now] = u[c] + kc
            X = X - X.max(axis=1, keepdims=True)
            E = np.exp(X)
            alpha = E / E.sum(axis=1, keepdims=True)
            y = alpha @ vc
            ga = gc[:, None] * alpha                       # d L / d v_i, per (t, i)
            if magnitude:
                ga = np.abs(ga)
                G = ga * (np.abs(vc)[None, :] + np.abs(y)[:, None])
            else:
                G = ga * (vc[None, :] - y[:, None])       # d L / d X[t,i]
            gv[bb, :, c] = ga.sum(axis=0)
            gk[bb, :, c] = G.sum(axis=0)
            gu[c] += np.trace(G)
            gw[c] += (1.0 if magnitude else -1.0) * (dist * G)[past].sum()
    return gk, gv, gw, gu
