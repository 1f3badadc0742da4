"""CPU fp64 oracle for the matrix-valued-state WKV of RWKV-5 "Eagle" and
RWKV-6 "Finch".

TEST INFRASTRUCTURE ONLY.  This module checks the HIP library; it is not part
of it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import, call or execute anything here.  It shares no
code with ``linear_attention_rnn_forward_amd`` and never imports it.

What it computes (vanos001.github.io, "RWKV (Attention-RNN Hybrid)", the
"Versions: RWKV-4 -> Eagle -> Finch" table and the matrix-form recurrence
under it): per batch row and head, with head dimension n (64 on the page),
a state S in R^{n x n} whose row index i runs over key channels and whose
column index j runs over value channels,

    S_t = diag(d_t) S_{t-1} + k_t v_t^T,        y_t = r_t^T S_t,

so y_t[j] = sum_i r_t[i] S_t[i, j].  The decay is d_t = exp(-softplus(z_t))
with z_t = a.b + w the page's decay argument: token-dependent for Finch, and
for Eagle (a state matrix with no data-dependent decay) the same function of
a per-channel z.  Channel c of a [B,T,C] tensor belongs to head c // n and
is index c % n inside it.  The initial state is zero unless one is passed.

Routines:

* ``softplus`` / ``decay`` -- log(1 + e^z) in the form that neither
  overflows nor cancels, and d = exp(-softplus(z)).
* ``forward`` -- the recurrence above, token by token, fp64.
* ``step`` -- one token of it over any leading shape (the decode form).
* ``direct`` -- the recurrence unrolled into its sum,
  y_t = sum_{s<=t} (sum_i r_t[i] k_s[i] prod_{s<tau<=t} d_tau[i]) v_s,
  with every decay product multiplied out term by term (O(T^3 n) per head;
  tiny T only).
* ``forward(..., magnitude=True)`` -- the same recurrence on |r|, |k|, |v|
  and |S_0|: the sum of the magnitudes of every term of every output, the
  scale against which the rounding of any evaluation order is measured.

Pins are in ``tests/test_oracle_matrix_pins.py``.  Inputs are promoted exactly
to fp64 from whatever they are stored as.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 64


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def softplus(z):
    """log(1 + e^z) = max(z, 0) + log1p(e^{-|z|}), fp64."""
    z = _f64(z)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def decay(z):
    """d = exp(-softplus(z)), the Finch decay of the page's table."""
    return np.exp(-softplus(z))


def _heads(x, n):
    """[..., C] -> [..., H, n]."""
    C = x.shape[-1]
    assert C % n == 0, f"C={C} is not a multiple of the head dimension {n}"
    return x.reshape(x.shape[:-1] + (C // n, n))


def _decay_per_token(z, B, T, C):
    z = _f64(z)
    if z.shape == (C,):
        return np.broadcast_to(decay(z), (B, T, C))
    assert z.shape == (B, T, C), f"z must be [C] or [B,T,C], got {z.shape}"
    return decay(z)


def forward(r, k, v, z, n=HEAD_DIM, state=None, magnitude=False):
    """The recurrence over [B,T,C]; returns (y [B,T,C], S_T [B,H,n,n]) in fp64.

    z is [C] (per channel, Eagle) or [B,T,C] (per token, Finch); state is
    None (zero) or [B,H,n,n].  magnitude=True runs it on |r|, |k|, |v|,
    |state| instead (see the module docstring).
    """
    r, k, v = _f64(r), _f64(k), _f64(v)
    B, T, C = k.shape
    assert r.shape == k.shape == v.shape
    H = C // n
    d = _decay_per_token(z, B, T, C)
    if magnitude:
        r, k, v = np.abs(r), np.abs(k), np.abs(v)
    S = np.zeros((B, H, n, n)) if state is None else _f64(state).reshape(B, H, n, n).copy()
    if magnitude:
        S = np.abs(S)
    y = np.empty((B, T, C))
    for t in range(T):
        S, y_t = _token(S, _heads(r[:, t], n), _heads(k[:, t], n), _heads(v[:, t], n),
                        _heads(d[:, t], n))
        y[:, t] = y_t.reshape(B, C)
    return y, S


def _token(S, r, k, v, d):
    """One application of the recurrence; every argument carries [..., H, n]
    (S [..., H, n, n])."""
    S = d[..., :, None] * S + k[..., :, None] * v[..., None, :]
    y = np.einsum("...i,...ij->...j", r, S)
    return S, y


def step(state, r, k, v, z, n=HEAD_DIM):
    """One token for every row of [..., C] (z the same shape as r, already
    broadcast by the caller); state [..., H, n, n].  Returns (y, S')."""
    r, k, v = _f64(r), _f64(k), _f64(v)
    lead = r.shape[:-1]
    C = r.shape[-1]
    S = _f64(state).reshape(lead + (C // n, n, n))
    S2, y = _token(S, _heads(r, n), _heads(k, n), _heads(v, n), _heads(decay(z), n))
    return y.reshape(lead + (C,)), S2


def direct(r, k, v, z, n=HEAD_DIM):
    """The unrolled sum from the zero state (tiny T only): for each head,
    W[t, s] = sum_i r_t[i] k_s[i] prod_{s<tau<=t} d_tau[i] for s <= t, and
    y_t = sum_s W[t, s] v_s.  The decay products are multiplied out factor by
    factor, not taken from cumulative sums."""
    r, k, v = _f64(r), _f64(k), _f64(v)
    B, T, C = k.shape
    H = C // n
    d = _decay_per_token(z, B, T, C)
    y = np.zeros((B, T, C))
    for b in range(B):
        for h in range(H):
            cs = slice(h * n, (h + 1) * n)
            R, K, V, D = r[b, :, cs], k[b, :, cs], v[b, :, cs], d[b, :, cs]
            W = np.zeros((T, T))
            for t in range(T):
                for s in range(t + 1):
                    prod = np.ones(n)
                    for tau in range(s + 1, t + 1):
                        prod = prod * D[tau]
                    W[t, s] = np.sum(R[t] * K[s] * prod)
            y[b, :, cs] = W @ V
    return y
