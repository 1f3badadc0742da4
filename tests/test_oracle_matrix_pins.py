"""Pins of the matrix-valued-state oracle (RWKV-5 Eagle / RWKV-6 Finch WKV:
S_t = diag(d_t) S_{t-1} + k_t v_t^T, y_t = r_t^T S_t, d_t = exp(-softplus(z_t));
vanos001.github.io "RWKV (Attention-RNN Hybrid)", the versions table and the
matrix-form recurrence under it).

The pages print no worked example for this variant, so the oracle is pinned
by what the recurrence fixes: its unrolled sum written independently, the
closed forms at the ends of the decay range (no decay: causal linear
attention, a plain matrix product; full decay: the current token only), the
one-channel case as a first-order IIR filter (scipy's lfilter), the decay
function against scipy's logistic function, and invariants (split and
resume, linearity, head permutation, the decode step chained over time).

Each pin is written as a check of a forward implementation, so the second
half of the file can show that plausible slips planted in copies of the
recurrence each fail at least one of them.
"""
import numpy as np
import pytest
import scipy.signal
import scipy.special

from oracle import matrix_state as ms


def _rand(seed, B, T, C, eagle=False):
    rng = np.random.default_rng(seed)
    r = rng.normal(0, 1, (B, T, C))
    k = rng.normal(0, 1, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    z = rng.normal(-1, 2, (C,) if eagle else (B, T, C))
    return r, k, v, z


def _oracle_fwd(r, k, v, z, n, state=None):
    return ms.forward(r, k, v, z, n=n, state=state)


# ---------------------------------------------------------------------------
# the pins, as checks of a forward implementation fwd(r, k, v, z, n, state)
# ---------------------------------------------------------------------------

def check_unrolled_sum(fwd):
    """The recurrence equals its unrolled sum (decay products multiplied out
    factor by factor), Finch and Eagle."""
    for seed, eagle in ((0, False), (1, True), (2, False)):
        r, k, v, z = _rand(seed, 2, 7, 8, eagle)
        y, _ = fwd(r, k, v, z, 4)
        yd = ms.direct(r, k, v, z, n=4)
        np.testing.assert_allclose(y, yd, rtol=1e-12, atol=1e-12)


def check_no_decay_is_linear_attention(fwd):
    """z -> -inf gives d = 1 exactly: y = tril(R K^T) V per head."""
    r, k, v, _ = _rand(3, 2, 9, 8)
    z = np.full((8,), -800.0)
    y, _ = fwd(r, k, v, z, 4)
    for b in range(2):
        for h in range(2):
            cs = slice(4 * h, 4 * h + 4)
            A = np.tril(r[b, :, cs] @ k[b, :, cs].T)
            np.testing.assert_allclose(y[b, :, cs], A @ v[b, :, cs], rtol=1e-12, atol=1e-12)


def check_full_decay_keeps_current_token(fwd):
    """z -> +inf gives d = 0 exactly: y_t = (r_t . k_t) v_t per head."""
    r, k, v, _ = _rand(4, 2, 6, 8)
    z = np.full((2, 6, 8), 800.0)
    y, _ = fwd(r, k, v, z, 4)
    for h in range(2):
        cs = slice(4 * h, 4 * h + 4)
        rk = np.sum(r[:, :, cs] * k[:, :, cs], axis=-1, keepdims=True)
        np.testing.assert_allclose(y[:, :, cs], rk * v[:, :, cs], rtol=1e-13, atol=1e-13)


def check_one_channel_is_iir_filter(fwd):
    """n = 1, per-channel decay d: S_t = d S_{t-1} + k_t v_t is the filter
    1 / (1 - d q^-1) applied to k v, and y_t = r_t S_t."""
    rng = np.random.default_rng(5)
    T, C = 40, 3
    r, k, v = (rng.normal(0, 1, (1, T, C)) for _ in range(3))
    z = rng.normal(0, 1.5, C)
    y, S = fwd(r, k, v, z, 1)
    for c in range(C):
        dc = scipy.special.expit(-z[c])
        s = scipy.signal.lfilter([1.0], [1.0, -dc], k[0, :, c] * v[0, :, c])
        np.testing.assert_allclose(y[0, :, c], r[0, :, c] * s, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S[0, c, 0, 0], s[-1], rtol=1e-12)


def check_finch_constant_equals_eagle(fwd):
    r, k, v, z = _rand(6, 2, 8, 8, eagle=True)
    y_e, S_e = fwd(r, k, v, z, 4)
    y_f, S_f = fwd(r, k, v, np.broadcast_to(z, (2, 8, 8)).copy(), 4)
    np.testing.assert_allclose(y_f, y_e, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(S_f, S_e, rtol=1e-14, atol=1e-14)


def check_split_and_resume(fwd):
    r, k, v, z = _rand(7, 2, 13, 8)
    y, S = fwd(r, k, v, z, 4)
    for cut in (1, 5, 12):
        y1, S1 = fwd(r[:, :cut], k[:, :cut], v[:, :cut], z[:, :cut], 4)
        y2, S2 = fwd(r[:, cut:], k[:, cut:], v[:, cut:], z[:, cut:], 4, state=S1)
        np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def check_linearity_and_heads(fwd):
    r, k, v, z = _rand(8, 2, 9, 12)
    v2 = np.random.default_rng(9).normal(0, 1, v.shape)
    y1, _ = fwd(r, k, v, z, 4)
    y2, _ = fwd(r, k, v2, z, 4)
    y12, _ = fwd(r, k, 2.5 * v - 0.75 * v2, z, 4)
    np.testing.assert_allclose(y12, 2.5 * y1 - 0.75 * y2, rtol=1e-11, atol=1e-11)
    yr, _ = fwd(-3.0 * r, k, v, z, 4)
    np.testing.assert_allclose(yr, -3.0 * y1, rtol=1e-12, atol=1e-12)
    # heads are independent: permuting them permutes the outputs
    perm = np.concatenate([np.arange(8, 12), np.arange(0, 4), np.arange(4, 8)])
    yp, _ = fwd(r[..., perm], k[..., perm], v[..., perm], z[..., perm], 4)
    np.testing.assert_allclose(yp, y1[..., perm], rtol=1e-13, atol=1e-13)


def check_first_token_from_a_state(fwd):
    """T = 1: y_0 = r_0^T (diag(d_0) S_0 + k_0 v_0^T)."""
    rng = np.random.default_rng(10)
    r, k, v = (rng.normal(0, 1, (1, 1, 4)) for _ in range(3))
    z = rng.normal(0, 1, (1, 1, 4))
    S0 = rng.normal(0, 1, (1, 1, 4, 4))
    y, S = fwd(r, k, v, z, 4, state=S0)
    d = scipy.special.expit(-z[0, 0])
    S_ref = d[:, None] * S0[0, 0] + np.outer(k[0, 0], v[0, 0])
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=1e-13)
    np.testing.assert_allclose(y[0, 0], r[0, 0] @ S_ref, rtol=1e-13, atol=1e-14)


PINS = [check_unrolled_sum, check_no_decay_is_linear_attention,
        check_full_decay_keeps_current_token, check_one_channel_is_iir_filter,
        check_finch_constant_equals_eagle, check_split_and_resume,
        check_linearity_and_heads, check_first_token_from_a_state]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(_oracle_fwd)


# ---------------------------------------------------------------------------
# pins that are not checks of the forward recurrence
# ---------------------------------------------------------------------------

def test_decay_is_the_logistic_of_minus_z():
    """exp(-softplus(z)) = 1 / (1 + e^z), scipy's expit(-z), over the whole
    range, including arguments where a literal log(1 + e^z) would overflow."""
    z = np.concatenate([np.linspace(-60, 60, 2401), [-1e3, -745.0, 700.0, 710.0, 1e3]])
    np.testing.assert_allclose(ms.decay(z), scipy.special.expit(-z), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(ms.softplus(z[np.abs(z) < 30]),
                               np.log1p(np.exp(z[np.abs(z) < 30])), rtol=1e-14)
    assert np.all(ms.decay(z) <= 1.0) and np.all(ms.decay(z) >= 0.0)


def test_step_chain_equals_forward():
    r, k, v, z = _rand(11, 2, 10, 8)
    y, S = ms.forward(r, k, v, z, n=4)
    st = np.zeros((2, 2, 4, 4))
    for t in range(10):
        y_t, st = ms.step(st, r[:, t], k[:, t], v[:, t], z[:, t], n=4)
        np.testing.assert_allclose(y_t, y[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(st, S, rtol=1e-13, atol=1e-13)


def test_magnitude_bounds_the_outputs():
    r, k, v, z = _rand(12, 2, 15, 8)
    S0 = np.random.default_rng(13).normal(0, 1, (2, 2, 4, 4))
    y, _ = ms.forward(r, k, v, z, n=4, state=S0)
    m, _ = ms.forward(r, k, v, z, n=4, state=S0, magnitude=True)
    assert np.all(m >= np.abs(y) - 1e-12)
    ya, _ = ms.forward(np.abs(r), np.abs(k), np.abs(v), z, n=4, state=np.abs(S0))
    np.testing.assert_allclose(m, ya, rtol=1e-14)


# ---------------------------------------------------------------------------
# plausible slips, planted in copies of the recurrence: each fails a pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def fwd(r, k, v, z, n, state=None):
        r, k, v = (np.asarray(a, dtype=np.float64) for a in (r, k, v))
        B, T, C = k.shape
        H = C // n
        zz = np.asarray(z, dtype=np.float64)
        if zz.shape == (C,):
            zz = np.broadcast_to(zz, (B, T, C))
        d = np.exp(-zz) if kind == "decay_exp_of_minus_z" else ms.decay(zz)
        S = np.zeros((B, H, n, n)) if state is None else np.array(state, dtype=np.float64)
        y = np.empty((B, T, C))
        for t in range(T):
            rt, kt, vt, dt = (a[:, t].reshape(B, H, n) for a in (r, k, v, d))
            if kind == "read_before_update":
                y[:, t] = np.einsum("bhi,bhij->bhj", rt, S).reshape(B, C)
            if kind == "decay_after_add":
                S = dt[..., :, None] * (S + kt[..., :, None] * vt[..., None, :])
            elif kind == "decay_on_value_index":
                S = S * dt[..., None, :] + kt[..., :, None] * vt[..., None, :]
            elif kind == "outer_product_transposed":
                S = dt[..., :, None] * S + vt[..., :, None] * kt[..., None, :]
            else:
                S = dt[..., :, None] * S + kt[..., :, None] * vt[..., None, :]
            if kind == "read_out_transposed":
                y[:, t] = np.einsum("bhj,bhij->bhi", rt, S).reshape(B, C)
            elif kind != "read_before_update":
                y[:, t] = np.einsum("bhi,bhij->bhj", rt, S).reshape(B, C)
        return y, S
    return fwd


MUTANTS = ["decay_after_add", "read_before_update", "outer_product_transposed",
           "decay_on_value_index", "read_out_transposed", "decay_exp_of_minus_z"]


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_each_planted_slip_fails_a_pin(kind):
    failed = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the slip {kind}"
